// Product-VQ encode / decode kernels for gfx950.
//
// Method ("Metal Kernels API" page, "VecInfer kernels",
// vecinfer_encode_decode_metal; "veloxquant_mlx.cache.vecinfer_cache module"
// page, module description): smooth (x / s) -> normalized Walsh-Hadamard
// rotation -> nearest centroid per sub-vector (squared L2, ties to the lowest
// index) -> [codebook gather -> inverse rotation -> x s].
//
// Layout on the wave: one lane per (token-head, sub-vector j).  The lane
// keeps its sub_dim values in registers; the rotation runs as an in-register
// butterfly over the low log2(sub_dim) index bits and as cross-lane
// butterflies (shuffles) over the high log2(D / sub_dim) bits, so a
// token-head's D values never leave the register file.  The nearest-centroid
// search walks the codebook with a wave-uniform centroid index, so every
// centroid read is a scalar (SGPR) load shared by the 64 lanes; distances
// and the running argmin stay in registers.
#include "vq_internal.h"
#include "vq_lane.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace vq {
namespace {

constexpr int kThreads = 256;  // 4 waves of 64
typedef float float4_t __attribute__((ext_vector_type(4)));  // 16x16 accumulator
// Workgroup size of a kernel whose waves split the codebook CSPLIT ways:
// one group of token-heads per workgroup when the codebook is split.
template <int CSPLIT>
constexpr int threads_for() { return CSPLIT > 4 ? 64 * CSPLIT : kThreads; }

struct Dims {
  int B, H, S, n_c, smooth_rows, transform, S_cap, S_off, use_row_offsets, recon_dtype;
  FastDiv div_S, div_H;  // by S and H (token-head indices below 2^31)
  int code_bits;         // 8, or 4: two codes per byte, the even sub-vector in the low nibble
};

// MODE 0: encode; 1: encode + reconstruct; 2: decode (codes_in -> recon);
// 3: forward transform only (fp32 (x / s) . H into recon, the vectors a
// codebook is trained on).
// CSPLIT waves share one group of token-heads and split the codebook between
// them (used when there are too few token-heads to fill the chip); their
// partial argmins are combined through LDS, lowest index first on ties.
// The body takes its workgroup index as an argument, so that one launch can
// run it for two inputs (the keys and the values of one append).
template <int D, int DS, int MODE, int CSPLIT>
__device__ __forceinline__ void pvq_body(
    int block, const __half* __restrict__ keys, const uint8_t* __restrict__ codes_in,
    const float* __restrict__ cb, const float* __restrict__ smooth,
    uint8_t* __restrict__ codes, void* __restrict__ recon, const Dims& d, const RowOffsets& offs) {
  constexpr int NSUB = D / DS;   // lanes per token-head (<= 64)
  constexpr int TPW = 64 / NSUB; // token-heads per wave
  constexpr int NT = threads_for<CSPLIT>();
  constexpr int TPB = (NT / 64 / CSPLIT) * TPW;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave / CSPLIT, part = wave % CSPLIT;
  const int j = lane % NSUB;
  // token-head indices are below 2^31 (checked on the host), so the index
  // arithmetic is 32-bit with the divisors' precomputed multipliers
  const uint32_t n_th = (uint32_t)d.B * (uint32_t)d.H * (uint32_t)d.S;
  const uint32_t th = (uint32_t)block * TPB + grp * TPW + lane / NSUB;
  const bool valid = th < n_th;
  const uint32_t th32 = valid ? th : 0u;
  const uint32_t bh32 = fast_div(th32, d.div_S);
  const uint32_t b32 = fast_div(bh32, d.div_H);
  const int t = (int)(th32 - bh32 * (uint32_t)d.S);
  const int h = (int)(bh32 - b32 * (uint32_t)d.H);
  const int b = (int)b32;
  const long long thc = th32, bh = bh32;
  const float* srow = smooth ? smooth + (long long)(d.smooth_rows == 1 ? 0 : h) * D + j * DS : nullptr;
  // the output slot's row offset (a kernel-argument array indexed by the
  // lane's batch row) is requested with the inputs, not after the search
  const int off = (MODE == 0 || MODE == 1) && d.use_row_offsets ? offs.v[b] : d.S_off;

  // The row's inputs (raw fp16 bits of the clamped row, smooth factors)
  // are requested before the codebook staging below, so all loads are in
  // flight together.
  float x[DS], sv[DS];
  RawHalves<DS> raw;
  if constexpr (MODE != 2) {
    raw = load_raw_f16<DS>(keys + thc * D + j * DS);
    if (srow) {
#pragma unroll
      for (int e = 0; e < DS; ++e) sv[e] = srow[e];
    }
  }

  // Short inputs (CSPLIT > 1) are latency bound: stage the codebook in LDS
  // with one coalesced pass (every load issued before any is stored)
  // instead of walking it with dependent scalar loads.
  const float* cbk = cb;
  if constexpr (CSPLIT > 1) {
    __shared__ float s_cb[256 * DS];
    constexpr int kPer = (256 * DS + NT - 1) / NT;
    float v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + k * NT;
      v[k] = i < d.n_c * DS ? cb[i] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + k * NT;
      if (i < 256 * DS) s_cb[i] = v[k];
    }
    __syncthreads();
    cbk = s_cb;
  }

  int idx = 0;
  if constexpr (MODE != 2) {
    cvt_raw_f16<DS>(raw, x);
    if (!valid) {
#pragma unroll
      for (int e = 0; e < DS; ++e) x[e] = 0.f;
    }
    if (srow) {
#pragma unroll
      for (int e = 0; e < DS; ++e) x[e] = x[e] / sv[e];
    }
    if (d.transform) wht<D, DS>(x, j);
    if constexpr (MODE == 3) {
      if (valid) store_f32<DS>(reinterpret_cast<float*>(recon) + thc * D + j * DS, x);
      return;
    }

    // Nearest centroid: fp32 squared distance summed over e in order,
    // strict '<' keeps the lowest index on exact ties.  The centroid index is
    // wave-uniform, so each centroid is one scalar load (or one LDS broadcast)
    // shared by all lanes.
    const int c_lo = d.n_c * part / CSPLIT, c_hi = d.n_c * (part + 1) / CSPLIT;
    float best = INFINITY;
    idx = c_lo;
#pragma unroll 8
    for (int c = c_lo; c < c_hi; ++c) {
      const float* cc = cbk + c * DS;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) {
        const float df = x[e] - cc[e];
        acc = fmaf(df, df, acc);
      }
      if (acc < best) { best = acc; idx = c; }
    }
    if constexpr (CSPLIT > 1) {
      __shared__ float s_best[NT];
      __shared__ int s_idx[NT];
      s_best[threadIdx.x] = best;
      s_idx[threadIdx.x] = idx;
      __syncthreads();
      if (part != 0) return;  // the first wave of the group finishes the token-heads
      // later parts hold higher indices: only a strictly smaller distance
      // wins (every partial is read before any is compared: no chain of
      // dependent LDS reads)
      float bk[CSPLIT];
      int ik[CSPLIT];
#pragma unroll
      for (int k = 1; k < CSPLIT; ++k) {
        bk[k] = s_best[threadIdx.x + k * 64];
        ik[k] = s_idx[threadIdx.x + k * 64];
      }
#pragma unroll
      for (int k = 1; k < CSPLIT; ++k) {
        const bool lt = bk[k] < best;
        best = lt ? bk[k] : best;
        idx = lt ? ik[k] : idx;
      }
    }
    // 4-bit codes: the even sub-vector's lane packs its odd neighbour's
    // code (lane + 1, the same token-head and the same row of 16 lanes: DPP
    // row_shl:1) into the high nibble
    const int idx_next = __builtin_amdgcn_mov_dpp(idx, 0x101, 0xf, 0xf, false);
    if (valid) {
      if (d.code_bits == 4) {
        if (!(j & 1))
          codes[(bh * d.S_cap + off + t) * (NSUB / 2) + j / 2] = (uint8_t)((idx & 15) | ((idx_next & 15) << 4));
      } else {
        codes[(bh * d.S_cap + off + t) * NSUB + j] = (uint8_t)idx;
      }
    }
  } else {
    if (valid) {
      int c;
      if (d.code_bits == 4) {
        const int byte = codes_in[(bh * d.S_cap + d.S_off + t) * (NSUB / 2) + j / 2];
        c = (j & 1) ? byte >> 4 : byte & 15;
      } else {
        c = codes_in[(bh * d.S_cap + d.S_off + t) * NSUB + j];
      }
      idx = min(c, d.n_c - 1);
    }
  }

  if constexpr (MODE == 1 || MODE == 2) {
    const float* cc = cbk + idx * DS;
#pragma unroll
    for (int e = 0; e < DS; ++e) x[e] = cc[e];
    if (d.transform) wht<D, DS>(x, j);  // H is its own inverse
    if (srow) {
#pragma unroll
      for (int e = 0; e < DS; ++e) x[e] = x[e] * srow[e];
    }
    if (valid) {
      if (d.recon_dtype == 1)
        store_f16<DS>(reinterpret_cast<__half*>(recon) + thc * D + j * DS, x);
      else
        store_f32<DS>(reinterpret_cast<float*>(recon) + thc * D + j * DS, x);
    }
  }
}

template <int D, int DS, int MODE, int CSPLIT>
__global__ __launch_bounds__(threads_for<CSPLIT>()) void pvq_kernel(
    const __half* __restrict__ keys, const uint8_t* __restrict__ codes_in,
    const float* __restrict__ cb, const float* __restrict__ smooth,
    uint8_t* __restrict__ codes, void* __restrict__ recon, Dims d, RowOffsets offs) {
  pvq_body<D, DS, MODE, CSPLIT>(blockIdx.x, keys, codes_in, cb, smooth, codes, recon, d, offs);
}

// ---------------------------------------------------------------------------
// Nearest centroid for rows of 8 on the matrix cores (the search of
// pvq_f16_kernel below, as helpers for the k-means and dense-matrix kernels):
// |c|^2 - 2 c.x on v_mfma_f32_32x32x8_f16 with each operand split into fp16
// high and low parts (three passes), the codebook scaled by 2^sc (largest
// |C| in [2^13, 2^14)) and a step's rows by the same scale unless they would
// leave the fp16 range (then their own scale, with rescaled norm seeds).
// Layout: lane l holds elements 4 (l / 32) + u of rows 32 g + l mod 32 of a
// 64-row step; candidates run in increasing index order, the lanes l and
// l ^ 32 holding the two halves of a tile merge lowest index first.
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

struct F16Codebook {
  half4_t ah[8 * 64], al[8 * 64];  // A operands [tile][lane], -2 C 2^sc hi and lo
  float norm[256];                 // |C 2^sc|^2, +inf past n_c
};

// Stage a codebook of up to 256 rows of 8: every thread of the workgroup
// (NT >= 256) takes part; ends with a barrier.  Returns sc.
template <int NT>
__device__ __forceinline__ int f16_stage(const float* __restrict__ cb, int n_c, F16Codebook& t,
                                         float* s_red) {
  constexpr int DS = 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  const int c = threadIdx.x;
  float m = 0.f;
  if (c < n_c) {
#pragma unroll
    for (int e = 0; e < DS; ++e) m = fmaxf(m, fabsf(cb[c * DS + e]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) m = fmaxf(m, s_red[w]);
  const int sc = m > 0.f ? 14 - __builtin_amdgcn_frexp_expf(m) : 0;
  if (c < 256) {
    float n = INFINITY;
    if (c < n_c) {
      n = 0.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) {
        const float v = ldexpf(cb[c * DS + e], sc);
        n = fmaf(v, v, n);
      }
    }
    t.norm[c] = n;
  }
  if (wave < 4) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int T = 2 * wave + r;
      const int cc = 32 * T + l32;
      half4_t ah, al;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float v = cc < n_c ? -2.f * ldexpf(cb[cc * DS + 4 * hi + u], sc) : 0.f;
        ah[u] = (_Float16)v;
        al[u] = (_Float16)(v - (float)ah[u]);
      }
      t.ah[T * 64 + lane] = ah;
      t.al[T * 64 + lane] = al;
    }
  }
  __syncthreads();
  return sc;
}

// Nearest centroids of the two rows a lane holds (idx[g]: row 32 g + l mod
// 32, the same in lanes l and l ^ 32).  seeded: this wave's 256 floats.
__device__ __forceinline__ void f16_nearest(const float (&x)[2][4], int sc, const F16Codebook& t,
                                            float* seeded, int n_c, int (&idx)[2]) {
  const int lane = threadIdx.x & 63;
  const int hi = lane >> 5;
  float mx = 0.f;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int u = 0; u < 4; ++u) mx = fmaxf(mx, fabsf(x[g][u]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  int s = sc;
  const float* nrm = t.norm;
  if (ldexpf(mx, sc) >= 32768.f) {
    s = 14 - __builtin_amdgcn_frexp_expf(mx);
    const float4 nv = *reinterpret_cast<const float4*>(t.norm + 4 * lane);
    const float f = ldexpf(1.f, s - sc);
    *reinterpret_cast<float4*>(seeded + 4 * lane) = make_float4(nv.x * f, nv.y * f, nv.z * f, nv.w * f);
    nrm = seeded;
  }
  half4_t bh[2], bl[2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float v = ldexpf(x[g][u], s);
      bh[g][u] = (_Float16)v;
      bl[g][u] = (_Float16)(v - (float)bh[g][u]);
    }
  struct TileIn {
    half4_t ah, al;
    float16_t n;
  };
  float best[2] = {INFINITY, INFINITY};
  int bi[2] = {0, 0}, bt[2] = {0, 0};
  auto tile_in = [&](int T) {
    asm volatile("" ::: "memory");
    TileIn ti;
    ti.ah = t.ah[T * 64 + lane];
    ti.al = t.al[T * 64 + lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 nv = *reinterpret_cast<const float4*>(nrm + 32 * T + 8 * q + 4 * hi);
      ti.n[4 * q] = nv.x; ti.n[4 * q + 1] = nv.y; ti.n[4 * q + 2] = nv.z; ti.n[4 * q + 3] = nv.w;
    }
    return ti;
  };
  auto chains = [&](const TileIn& ti, float16_t (&a)[2]) {
    a[0] = __builtin_amdgcn_mfma_f32_32x32x8f16(ti.ah, bh[0], ti.n, 0, 0, 0);
    a[1] = __builtin_amdgcn_mfma_f32_32x32x8f16(ti.ah, bh[1], ti.n, 0, 0, 0);
    a[0] = __builtin_amdgcn_mfma_f32_32x32x8f16(ti.al, bh[0], a[0], 0, 0, 0);
    a[1] = __builtin_amdgcn_mfma_f32_32x32x8f16(ti.al, bh[1], a[1], 0, 0, 0);
    a[0] = __builtin_amdgcn_mfma_f32_32x32x8f16(ti.ah, bl[0], a[0], 0, 0, 0);
    a[1] = __builtin_amdgcn_mfma_f32_32x32x8f16(ti.ah, bl[1], a[1], 0, 0, 0);
  };
  auto scan = [&](const float16_t (&r)[2], int T) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float before = best[g];
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (r[g][v] < best[g]) { best[g] = r[g][v]; bi[g] = 8 * (v >> 2) + (v & 3); }
      if (best[g] < before) bt[g] = T;
    }
  };
  float16_t a[2];
  chains(tile_in(0), a);
  TileIn nxt_in = tile_in(1);
#pragma unroll
  for (int T = 0; T < 8; ++T) {
    float16_t r[2] = {a[0], a[1]};
    if (T + 1 < 8) {
      chains(nxt_in, a);
      if (T + 2 < 8) nxt_in = tile_in(T + 2);
    }
    scan(r, T);
#pragma unroll
    for (int g = 0; g < 2; ++g)
      asm volatile("" : "+v"(best[g]), "+v"(bi[g]), "+v"(bt[g]), "+v"(a[g]));
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float bv = best[g];
    int bx = 32 * bt[g] + bi[g] + 4 * hi;
    const float ov = __shfl_xor(bv, 32);
    const int ox = __shfl_xor(bx, 32);
    if (ov < bv || (ov == bv && ox < bx)) bx = ox;
    idx[g] = min(bx, n_c - 1);
  }
}

// Dense rotation (transform == 2): an explicit invertible [D, D] matrix M,
// the H_mat argument of vecinfer_encode_decode_metal ("Metal Kernels API",
// "VecInfer kernels"): encode rotates x / s by M (x~ = (x / s) . M, a row
// vector times M), decode by M^-1.  One lane per (token-head, sub-vector j)
// as in pvq_body; the token-head's D values are staged in LDS and the lane
// forms its sub_dim outputs y[e] = sum_i x[i] A[i][j d + e] with the
// matrix A held in LDS for the whole (grid-stride) launch.  fp32 products
// summed in index order; then the same nearest-centroid search.
template <int D, int DS, int MODE, int NT>
__global__ __launch_bounds__(NT) void pvq_dense_kernel(
    const __half* __restrict__ keys, const uint8_t* __restrict__ codes_in,
    const float* __restrict__ cb, const float* __restrict__ smooth,
    const float* __restrict__ rot, const float* __restrict__ rot_inv,
    uint8_t* __restrict__ codes, void* __restrict__ recon, Dims d, RowOffsets offs) {
  constexpr int NSUB = D / DS;      // lanes per token-head
  constexpr int TPW = 64 / NSUB;    // token-heads per wave step
  constexpr int WPB = NT / 64;
  constexpr int NMAT = MODE == 1 ? 2 : 1;  // M (encode), M^-1 (decode), or both
  // sub-vectors of 8 with 8-bit codes: the nearest centroid on the matrix
  // cores (f16_nearest), after moving the rows into its lane layout
  constexpr bool kMF = DS == 8 && (MODE == 0 || MODE == 1);
  __shared__ std::conditional_t<kMF, F16Codebook, char> tab;
  __shared__ float s_red[WPB];
  __shared__ std::conditional_t<kMF, float[WPB][256], char> s_seeded;
  extern __shared__ __align__(16) float dl[];
  float* const mat = dl;                          // [NMAT][D][D]
  float* const xs = dl + NMAT * D * D;            // [WPB][TPW][D] staged vectors
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane % NSUB, tok = lane / NSUB;
  {
    const float* src0 = MODE == 2 ? rot_inv : rot;
    for (int i = threadIdx.x; i < D * D / 4; i += NT)
      reinterpret_cast<float4*>(mat)[i] = reinterpret_cast<const float4*>(src0)[i];
    if constexpr (MODE == 1)
      for (int i = threadIdx.x; i < D * D / 4; i += NT)
        reinterpret_cast<float4*>(mat + D * D)[i] = reinterpret_cast<const float4*>(rot_inv)[i];
  }
  __syncthreads();
  int sc = 0;
  if constexpr (kMF) {
    if (d.code_bits == 8) sc = f16_stage<NT>(cb, d.n_c, tab, s_red);
  }
  float* const xw = xs + (wave * TPW + tok) * D;  // this lane's token-head vector
  // y = x . A for the lane's sub-vector: x staged in xw (the wave's own LDS
  // accesses execute in issue order, so the reads see the writes)
  // For sub-vectors of 8, lanes j and j + 8 of a token-head would read the
  // same bank quads of a matrix row (32 B apart per lane): lanes with bit 3
  // of j set read the row's two halves in the other order and accumulate
  // them swapped, undone once at the end.
  const bool swap = DS == 8 && ((j >> 3) & 1);
  auto rotate = [&](float (&x)[DS], const float* A) {
#pragma unroll
    for (int e = 0; e < DS; ++e) xw[j * DS + e] = x[e];
    float y[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) y[e] = 0.f;
    const int h0 = swap ? 4 : 0;
    for (int i = 0; i < D; i += 4) {
      const float4 xv = *reinterpret_cast<const float4*>(xw + i);
      const float xi[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float* arow = A + (i + k) * D + j * DS;
        if constexpr (DS == 8) {
          const float4 a0 = *reinterpret_cast<const float4*>(arow + h0);
          const float4 a1 = *reinterpret_cast<const float4*>(arow + (4 - h0));
          const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
          for (int e = 0; e < DS; ++e) y[e] = fmaf(xi[k], av[e], y[e]);
        } else {
#pragma unroll
          for (int e = 0; e < DS; ++e) y[e] = fmaf(xi[k], arow[e], y[e]);
        }
      }
    }
    if constexpr (DS == 8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = swap ? y[4 + e] : y[e];
        x[4 + e] = swap ? y[e] : y[4 + e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < DS; ++e) x[e] = y[e];
    }
  };

  const long long n_th = (long long)d.B * d.H * d.S;
  const long long n_steps = (n_th + TPW - 1) / TPW;
  for (long long step = (long long)blockIdx.x * WPB + wave; step < n_steps;
       step += (long long)gridDim.x * WPB) {
    const long long th = step * TPW + tok;
    const bool valid = th < n_th;
    const long long thc = valid ? th : 0;
    const int t = (int)(thc % d.S);
    const long long bh = thc / d.S;
    const int h = (int)(bh % d.H);
    const int b = (int)(bh / d.H);
    const float* srow =
        smooth ? smooth + (long long)(d.smooth_rows == 1 ? 0 : h) * D + j * DS : nullptr;
    float x[DS];
    int idx = 0;
    if constexpr (MODE != 2) {
      RawHalves<DS> raw = load_raw_f16<DS>(keys + thc * D + j * DS);
      cvt_raw_f16<DS>(raw, x);
      if (!valid) {
#pragma unroll
        for (int e = 0; e < DS; ++e) x[e] = 0.f;
      }
      if (srow) {
#pragma unroll
        for (int e = 0; e < DS; ++e) x[e] = x[e] / srow[e];
      }
      rotate(x, mat);
      if constexpr (MODE == 3) {
        if (valid) store_f32<DS>(reinterpret_cast<float*>(recon) + thc * D + j * DS, x);
        continue;
      }
      bool searched = false;
      if constexpr (kMF) {
        if (d.code_bits == 8) {
          // row r of the step is lane r; the matrix-core layout wants
          // elements 4 (l / 32) + u of rows 32 g + l mod 32 in lane l
          const int hi = lane >> 5, l32 = lane & 31;
          float xm[2][4];
#pragma unroll
          for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float lo_v = __shfl(x[u], 32 * g + l32);
              const float hi_v = __shfl(x[4 + u], 32 * g + l32);
              xm[g][u] = hi ? hi_v : lo_v;
            }
          int ids[2];
          f16_nearest(xm, sc, tab, s_seeded[wave], d.n_c, ids);
          idx = hi ? ids[1] : ids[0];
          searched = true;
        }
      }
      if (!searched) {
        // nearest centroid (fp32 squared distance over e in order, strict '<')
        float best = INFINITY;
#pragma unroll 8
        for (int c = 0; c < d.n_c; ++c) {
          const float* cc = cb + c * DS;
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < DS; ++e) {
            const float df = x[e] - cc[e];
            acc = fmaf(df, df, acc);
          }
          if (acc < best) { best = acc; idx = c; }
        }
      }
      const int idx_next = __shfl_down(idx, 1);
      if (valid) {
        const int off = d.use_row_offsets ? offs.v[b] : d.S_off;
        if (d.code_bits == 4) {
          if (!(j & 1))
            codes[(bh * d.S_cap + off + t) * (NSUB / 2) + j / 2] = (uint8_t)((idx & 15) | ((idx_next & 15) << 4));
        } else {
          codes[(bh * d.S_cap + off + t) * NSUB + j] = (uint8_t)idx;
        }
      }
    } else {
      if (valid) {
        int c;
        if (d.code_bits == 4) {
          const int byte = codes_in[(bh * d.S_cap + d.S_off + t) * (NSUB / 2) + j / 2];
          c = (j & 1) ? byte >> 4 : byte & 15;
        } else {
          c = codes_in[(bh * d.S_cap + d.S_off + t) * NSUB + j];
        }
        idx = min(c, d.n_c - 1);
      }
    }
    if constexpr (MODE == 1 || MODE == 2) {
      const float* cc = cb + idx * DS;
#pragma unroll
      for (int e = 0; e < DS; ++e) x[e] = cc[e];
      rotate(x, MODE == 1 ? mat + D * D : mat);  // by M^-1
      if (srow) {
#pragma unroll
        for (int e = 0; e < DS; ++e) x[e] = x[e] * srow[e];
      }
      if (valid) {
        if (d.recon_dtype == 1)
          store_f16<DS>(reinterpret_cast<__half*>(recon) + thc * D + j * DS, x);
        else
          store_f32<DS>(reinterpret_cast<float*>(recon) + thc * D + j * DS, x);
      }
    }
  }
}

// Encode of the keys and the values of one append in one launch (the cache
// appends both, "veloxquant_mlx.cache.vecinfer_cache module",
// update_and_fetch): workgroups [0, k_blocks) encode the keys with their
// smoothing and rotation, the rest the values.  For short appends, whose
// time is the latency of a few dependent memory round trips, the two halves
// then overlap instead of running one after the other.
template <int D, int DSK, int DSV, int CSPLIT>
__global__ __launch_bounds__(threads_for<CSPLIT>()) void pvq_kv_kernel(
    const __half* __restrict__ keys, const __half* __restrict__ values,
    const float* __restrict__ k_cb, const float* __restrict__ v_cb, const float* __restrict__ smooth,
    uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes, Dims dk, Dims dv,
    RowOffsets offs, int k_blocks) {
  if ((int)blockIdx.x < k_blocks)
    pvq_body<D, DSK, 0, CSPLIT>(blockIdx.x, keys, nullptr, k_cb, smooth, k_codes, nullptr, dk, offs);
  else
    pvq_body<D, DSV, 0, CSPLIT>(blockIdx.x - k_blocks, values, nullptr, v_cb, nullptr, v_codes, nullptr,
                                dv, offs);
}

// Encode of one token-head by a workgroup of 4 waves, for appends of a few
// token-heads (one new token per row of a decode step): the search is
// spread over many workgroups instead of the waves of a few, whose shared
// SIMDs would serialize it.  Lane (replica r, sub-vector j) of wave w holds
// the token-head's sub-vector j (every wave and replica computes the same
// smoothing and rotation) and scans the centroids c = p, p + P, p + 2 P, ...
// of part p = R w + r (R = 64 / NSUB replicas per wave, P = 4 R parts), with
// the fp32 squared distance summed over e in order and a strict '<'.  The P
// partial minima merge as (distance, index) pairs, so the result is the
// lowest index among the centroids at the minimal distance: the sequential
// search's answer.
template <int D, int DS>
__device__ __forceinline__ void pvq_short_body(
    uint32_t th, const __half* __restrict__ keys, const float* __restrict__ cb,
    const float* __restrict__ smooth, uint8_t* __restrict__ codes, const Dims& d,
    const RowOffsets& offs) {
  constexpr int NSUB = D / DS;  // sub-vectors per token-head (<= 64)
  constexpr int R = 64 / NSUB;  // replicas per wave
  constexpr int P = 4 * R;      // parts of the codebook
  static_assert(NSUB <= 64 && 64 % NSUB == 0 && 256 * DS % (4 * kThreads) == 0, "layout");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane % NSUB;
  const int part = R * wave + lane / NSUB;
  const uint32_t bh = fast_div(th, d.div_S);
  const uint32_t b = fast_div(bh, d.div_H);
  const int t = (int)(th - bh * (uint32_t)d.S);
  const int h = (int)(bh - b * (uint32_t)d.H);
  const float* srow = smooth ? smooth + (d.smooth_rows == 1 ? 0 : h) * D + j * DS : nullptr;
  const int off = d.use_row_offsets ? offs.v[b] : d.S_off;

  // the row's inputs and the codebook (zero rows past n_c) are requested
  // together
  const RawHalves<DS> raw = load_raw_f16<DS>(keys + (size_t)th * D + j * DS);
  float sv[DS];
  if (srow) {
#pragma unroll
    for (int e = 0; e < DS; ++e) sv[e] = srow[e];
  }
  __shared__ float s_cb[256 * DS];
  __shared__ float s_best[kThreads];
  __shared__ int s_idx[kThreads];
  {
    constexpr int kPer = 256 * DS / (4 * kThreads);  // float4 per thread
    float4 v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + k * kThreads;  // float4 index
      v[k] = 4 * i < d.n_c * DS ? reinterpret_cast<const float4*>(cb)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) reinterpret_cast<float4*>(s_cb)[threadIdx.x + k * kThreads] = v[k];
  }
  __syncthreads();

  float x[DS];
  cvt_raw_f16<DS>(raw, x);
  if (srow) {
#pragma unroll
    for (int e = 0; e < DS; ++e) x[e] = x[e] / sv[e];
  }
  if (d.transform) wht<D, DS>(x, j);

  float best = INFINITY;
  int idx = part < d.n_c ? part : 0x7fffffff;
  for (int c = part; c < d.n_c; c += P) {
    const float* cc = s_cb + c * DS;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < DS; ++e) {
      const float df = x[e] - cc[e];
      acc = fmaf(df, df, acc);
    }
    if (acc < best) { best = acc; idx = c; }
  }
  s_best[threadIdx.x] = best;
  s_idx[threadIdx.x] = idx;
  __syncthreads();
  if (wave != 0 || lane >= NSUB) return;
  // lane j of wave 0 merges the P parts of sub-vector j (every partial is
  // read before any is compared)
  float bk[P];
  int ik[P];
#pragma unroll
  for (int k = 1; k < P; ++k) {
    const int src = 64 * (k / R) + NSUB * (k % R) + j;  // part k
    bk[k] = s_best[src];
    ik[k] = s_idx[src];
  }
#pragma unroll
  for (int k = 1; k < P; ++k) {
    const bool lt = bk[k] < best || (bk[k] == best && ik[k] < idx);
    best = lt ? bk[k] : best;
    idx = lt ? ik[k] : idx;
  }
  // 4-bit codes: the even sub-vector's lane packs its odd neighbour's code
  // (lane + 1, the same row of 16 lanes: DPP row_shl:1) into the high nibble
  const int idx_next = __builtin_amdgcn_mov_dpp(idx, 0x101, 0xf, 0xf, false);
  const size_t slot = (size_t)bh * d.S_cap + off + t;
  if (d.code_bits == 4) {
    if (!(j & 1)) codes[slot * (NSUB / 2) + j / 2] = (uint8_t)((idx & 15) | ((idx_next & 15) << 4));
  } else {
    codes[slot * NSUB + j] = (uint8_t)idx;
  }
}

// The keys (workgroups [0, n_th)) and the values (the rest) of a short
// append, one token-head per workgroup.
template <int D, int DSK, int DSV>
__global__ __launch_bounds__(kThreads) void pvq_short_kv_kernel(
    const __half* __restrict__ keys, const __half* __restrict__ values,
    const float* __restrict__ k_cb, const float* __restrict__ v_cb, const float* __restrict__ smooth,
    uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes, Dims dk, Dims dv,
    RowOffsets offs, uint32_t n_th) {
  if (blockIdx.x < n_th)
    pvq_short_body<D, DSK>(blockIdx.x, keys, k_cb, smooth, k_codes, dk, offs);
  else
    pvq_short_body<D, DSV>(blockIdx.x - n_th, values, v_cb, nullptr, v_codes, dv, offs);
}

// Nearest centroid as a dense contraction on the matrix cores.  For a
// sub-vector x, |x - c|^2 = |x|^2 + (|c|^2 - 2 c.x), and |x|^2 is the same
// for every centroid, so the argmin over c of |c|^2 - 2 c.x is the argmin of
// the distance.  The contraction runs on v_mfma_f32_16x16x4_f32 (fp32
// operands and accumulation): A = the codebook scaled by -2 (16 centroids
// per tile, k = element), B = 16 sub-vectors, C starts from |c|^2.
//
// Layout: a wave step covers 64 sub-vector rows as four 16-row column groups
// cg; lane l holds, for every cg, elements 4 i + l / 16 (i < DS / 4) of row
// 16 cg + l mod 16, which is the B operand layout.  The rows' inputs are
// loaded straight into it and the rotation runs in it: element bits 0-1 are
// lane bits 4-5, the higher element bits are i, sub-vector bits 0-3 are lane
// bits 0-3 and sub-vector bits 4-5 (32 or 64 sub-vectors per head) are cg.
// The accumulator of tile T gives lane l the centroids 16 T + 4 (l / 16) + v
// (v < 4) of its row; each lane keeps a running argmin over them in
// increasing index order, and the four lanes of a row are merged at the end
// (lowest index on ties).
template <int D, int DS>
__device__ __forceinline__ void wht_b(float (&x)[4][DS / 4], int lane) {
  constexpr int NE = DS / 4;
  constexpr int NSUB = D / DS;
  constexpr int JL = NSUB < 16 ? NSUB : 16;  // sub-vector index range held in lane bits 0-3
  // butterfly over a lane bit m: (lo, hi) -> (lo + hi, lo - hi)
  auto lane_stage = [&](int m) {
    const float sg = (lane & m) ? -1.f : 1.f;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        const float y = __shfl_xor(x[cg][i], m);
        x[cg][i] = fmaf(sg, x[cg][i], y);
      }
  };
  lane_stage(16);
  lane_stage(32);
#pragma unroll
  for (int hb = 1; hb < NE; hb <<= 1)
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
#pragma unroll
      for (int i = 0; i < NE; ++i)
        if (!(i & hb)) {
          const float a = x[cg][i], b = x[cg][i | hb];
          x[cg][i] = a + b;
          x[cg][i | hb] = a - b;
        }
#pragma unroll
  for (int m = 1; m < JL; m <<= 1) lane_stage(m);
#pragma unroll
  for (int hb = 1; hb < NSUB / 16; hb <<= 1)
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
      if (!(cg & hb)) {
#pragma unroll
        for (int i = 0; i < NE; ++i) {
          const float a = x[cg][i], b = x[cg | hb][i];
          x[cg][i] = a + b;
          x[cg | hb][i] = a - b;
        }
      }
  const float nrm = WhtNorm<D>::value;
#pragma unroll
  for (int cg = 0; cg < 4; ++cg)
#pragma unroll
    for (int i = 0; i < NE; ++i) x[cg][i] *= nrm;
}

template <int D, int DS, int MODE>
__global__ __launch_bounds__(kThreads) void pvq_mfma_kernel(
    const __half* __restrict__ keys, const float* __restrict__ cb, const float* __restrict__ smooth,
    uint8_t* __restrict__ codes, void* __restrict__ recon, Dims d, RowOffsets offs) {
  static_assert(DS % 4 == 0 && DS <= 16, "K steps of 4 elements");
  constexpr int NSUB = D / DS;   // rows per token-head (<= 64)
  constexpr int TPW = 64 / NSUB; // token-heads per wave step
  constexpr int NE = DS / 4;     // matrix steps per tile and column group
  constexpr int WPB = kThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4, jl = lane & 15;

  // LDS: A operands per tile ([T][lane][i] = -2 C[16 T + lane mod 16][4 i +
  // lane / 16], zero past n_c) and |c|^2 (summed over e in order; +inf past
  // n_c, so the padding to 16 tiles never wins a strict '<')
  __shared__ float s_a[16 * 64 * NE];
  __shared__ float s_norm[256];
  {
    const int c = threadIdx.x;
    float n = INFINITY;
    if (c < d.n_c) {
      n = 0.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) n = fmaf(cb[c * DS + e], cb[c * DS + e], n);
    }
    s_norm[c] = n;
#pragma unroll
    for (int r = 0; r < 4 * NE; ++r) {
      const int idx = threadIdx.x + kThreads * r;          // [T][lane][i]
      const int T = idx / (64 * NE), ln = (idx / NE) % 64, ii = idx % NE;
      const int cc = 16 * T + (ln & 15);
      s_a[idx] = cc < d.n_c ? -2.f * cb[cc * DS + 4 * ii + (ln >> 4)] : 0.f;
    }
  }

  const int n_th = d.B * d.H * d.S;  // below 2^31 (the launcher checks)
  const int n_steps = (n_th + TPW - 1) / TPW;
  const int stride = (int)gridDim.x * WPB;

  // Row 16 cg + jl of the step starting at token-head th0: token-head
  // th0 + (16 cg + jl) / NSUB, sub-vector (16 cg + jl) mod NSUB.
  auto th_of = [&](int th0, int cg) { return th0 + (16 * cg + jl) / NSUB; };
  auto j_of = [&](int cg) { return (16 * cg + jl) % NSUB; };

  uint16_t raw[4][NE];
  float sv[4][NE];
  auto load_rows = [&](int th0) {
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
      int th = th_of(th0, cg);
      th = th < n_th ? th : 0;
      const uint16_t* p =
          reinterpret_cast<const uint16_t*>(keys) + (long long)th * D + j_of(cg) * DS + q;
#pragma unroll
      for (int i = 0; i < NE; ++i) raw[cg][i] = p[4 * i];
      if (smooth) {
        const int bh = (int)fast_div((uint32_t)th, d.div_S);
        const int h = d.smooth_rows == 1 ? 0 : bh - (int)fast_div((uint32_t)bh, d.div_H) * d.H;
        const float* sp = smooth + h * D + j_of(cg) * DS + q;
#pragma unroll
        for (int i = 0; i < NE; ++i) sv[cg][i] = sp[4 * i];
      }
    }
  };

  int step = (int)blockIdx.x * WPB + wave;
  load_rows((step < n_steps ? step : 0) * TPW);
  __syncthreads();

  for (; step < n_steps; step += stride) {
    const int th0 = step * TPW;
    float x[4][NE];
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        const uint16_t bits = raw[cg][i];
        float v = th_of(th0, cg) < n_th ? __half2float(*reinterpret_cast<const __half*>(&bits)) : 0.f;
        // x / s as x * rcp(s) (within 2 ulp of the quotient; such a
        // difference can only move a code at a near-tie)
        if (smooth) v = v * __builtin_amdgcn_rcpf(sv[cg][i]);
        x[cg][i] = v;
      }
    float svc[4][NE];  // this step's smooth factors, for the reconstruction
    if constexpr (MODE == 1) {
      if (smooth) {
#pragma unroll
        for (int cg = 0; cg < 4; ++cg)
#pragma unroll
          for (int i = 0; i < NE; ++i) svc[cg][i] = sv[cg][i];
      }
    }
    // the next step's inputs are requested now and consumed next iteration
    load_rows((step + stride < n_steps ? step + stride : step) * TPW);
    if (d.transform) wht_b<D, DS>(x, lane);

    // Tiles in order: stage T issues the matrix steps of tile T + 1 (all
    // column groups; A and |c|^2 read from LDS one stage earlier) between the
    // argmin updates of tile T.
    struct TileIn {
      float a[NE];
      float4_t n;
    };
    auto tile_in = [&](int T) {
      // re-read per stage (a compiler barrier keeps the 16 tiles' operands
      // from being hoisted out of the step loop into live registers)
      asm volatile("" ::: "memory");
      TileIn t;
      const float* ap = s_a + (T * 64 + lane) * NE;
#pragma unroll
      for (int i = 0; i < NE; ++i) t.a[i] = ap[i];
      const float4 nv = *reinterpret_cast<const float4*>(s_norm + 16 * T + 4 * q);
      t.n = float4_t{nv.x, nv.y, nv.z, nv.w};
      return t;
    };
    auto chains = [&](const TileIn& t, float4_t (&acc)[4]) {
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        acc[cg] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.a[0], x[cg][0], t.n, 0, 0, 0);
#pragma unroll
        for (int i = 1; i < NE; ++i)
          acc[cg] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.a[i], x[cg][i], acc[cg], 0, 0, 0);
      }
    };
    float best[4];
    int bi[4];
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) { best[cg] = INFINITY; bi[cg] = 0; }
    // kv[v] = 16 T + v for the tile being scanned, in registers the compiler
    // cannot fold into constants: indices above 64 are no inline constants,
    // and as literals they would be held in 256 registers across the loop
    int kv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) asm volatile("v_mov_b32 %0, %1" : "=v"(kv[v]) : "n"(v));
    auto scan = [&](const float4_t (&r)[4]) {
#pragma unroll
      for (int cg = 0; cg < 4; ++cg)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (r[cg][v] < best[cg]) { best[cg] = r[cg][v]; bi[cg] = kv[v]; }
#pragma unroll
      for (int v = 0; v < 4; ++v) kv[v] += 16;
    };
    float4_t acc[4];
    chains(tile_in(0), acc);
    TileIn nxt_in = tile_in(1);
#pragma unroll
    for (int T = 0; T < 16; ++T) {
      float4_t r[4];
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) r[cg] = acc[cg];
      if (T + 1 < 16) {
        chains(nxt_in, acc);
        if (T + 2 < 16) nxt_in = tile_in(T + 2);
      }
      scan(r);
      // Pin the stage in program order (IR passes otherwise regroup the
      // independent argmin chains by column group across all tiles, keeping
      // every tile's accumulators live): the argmin state of tile T and the
      // accumulators of tile T + 1 are materialized here.
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) asm volatile("" : "+v"(best[cg]), "+v"(bi[cg]), "+v"(acc[cg]));
      __builtin_amdgcn_sched_barrier(0);
    }

    // merge the four lanes of each row (lane bits 4-5), lowest index on ties
    int idx[4];
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
      float bv = best[cg];
      int bx = bi[cg] + 4 * q;
#pragma unroll
      for (int m = 16; m <= 32; m <<= 1) {
        const float ov = __shfl_xor(bv, m);
        const int ox = __shfl_xor(bx, m);
        if (ov < bv || (ov == bv && ox < bx)) { bv = ov; bx = ox; }
      }
      // (a row that never compares below +inf, e.g. NaN input, keeps a start index)
      idx[cg] = min(bx, d.n_c - 1);
    }

    // lane l writes the code of row (cg = l / 16, l mod 16)
    {
      const int code = q == 0 ? idx[0] : (q == 1 ? idx[1] : (q == 2 ? idx[2] : idx[3]));
      const int th = th0 + (16 * q + jl) / NSUB;
      if (th < n_th) {
        const int bh = (int)fast_div((uint32_t)th, d.div_S);
        const int t = th - bh * d.S;
        const int off = d.use_row_offsets ? offs.v[fast_div((uint32_t)bh, d.div_H)] : d.S_off;
        codes[((long long)bh * d.S_cap + off + t) * NSUB + (16 * q + jl) % NSUB] = (uint8_t)code;
      }
    }
    if constexpr (MODE == 1) {
#pragma unroll
      for (int cg = 0; cg < 4; ++cg)
#pragma unroll
        for (int i = 0; i < NE; ++i) x[cg][i] = cb[idx[cg] * DS + 4 * i + q];
      if (d.transform) wht_b<D, DS>(x, lane);  // H is its own inverse
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        const int th = th_of(th0, cg);
        if (th >= n_th) continue;
        const long long base = (long long)th * D + j_of(cg) * DS + q;
#pragma unroll
        for (int i = 0; i < NE; ++i) {
          const float v = smooth ? x[cg][i] * svc[cg][i] : x[cg][i];
          if (d.recon_dtype == 1)
            reinterpret_cast<__half*>(recon)[base + 4 * i] = __float2half_rn(v);
          else
            reinterpret_cast<float*>(recon)[base + 4 * i] = v;
        }
      }
    }
  }
}

// Sub-vectors of 8: the same search on v_mfma_f32_32x32x8_f16, whose K of
// 8 is one sub-vector, with each fp32 operand split into two fp16 parts
// (hi = fp16(v), lo = fp16(v - hi)) and three passes hi.hi + lo.hi + hi.lo
// (the dropped lo.lo term is below 2^-22 of the product).  Operands are
// scaled by powers of two first: the codebook by 2^sc (largest magnitude in
// [2^13, 2^14)), the sub-vectors of a step by the same 2^sc, so |c|^2 2^2sc
// seeds the accumulator unchanged; a step whose values would leave the fp16
// range at that scale takes its own 2^s and seeds with |c|^2 2^(s + sc)
// (both forms are 2^(s + sc) (|c|^2 - 2 c.x), whose argmin is the same).
//
// Layout: a wave step covers 64 rows as two 32-row column groups g; lane l
// holds elements 4 (l / 32) + u (u < 4) of row 32 g + l mod 32 (the B
// operand), loaded as 8 contiguous bytes and rotated in place: element bits
// 0-1 are u, element bit 2 is lane bit 5, sub-vector bits are lane bits 0-4.
// Tile T gives lane l the centroids 32 T + 8 (v / 4) + 4 (l / 32) + v mod 4
// (v < 16) of its row; lanes l and l ^ 32 hold the two halves.
template <int D>
__device__ __forceinline__ void wht_b8(float (&x)[2][4], int lane) {
  constexpr int NSUB = D / 8;  // 4..32: sub-vector bits are lane bits 0..4
#pragma unroll
  for (int g = 0; g < 2; ++g) {
#pragma unroll
    for (int hb = 1; hb < 4; hb <<= 1)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (!(u & hb)) {
          const float a = x[g][u], b = x[g][u | hb];
          x[g][u] = a + b;
          x[g][u | hb] = a - b;
        }
  }
  auto lane_stage = [&](int m) {
    const float sg = (lane & m) ? -1.f : 1.f;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) x[g][u] = fmaf(sg, x[g][u], __shfl_xor(x[g][u], m));
  };
  lane_stage(32);
#pragma unroll
  for (int m = 1; m < NSUB; m <<= 1) lane_stage(m);
  const float nrm = WhtNorm<D>::value;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int u = 0; u < 4; ++u) x[g][u] *= nrm;
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void pvq_f16_kernel(
    const __half* __restrict__ keys, const float* __restrict__ cb, const float* __restrict__ smooth,
    uint8_t* __restrict__ codes, void* __restrict__ recon, Dims d, RowOffsets offs) {
  constexpr int DS = 8;
  constexpr int NSUB = D / DS;   // rows per token-head (4..32)
  constexpr int TPW = 64 / NSUB; // token-heads per wave step
  constexpr int WPB = kThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hi = lane >> 5, l32 = lane & 31;

  // codebook scale 2^sc: the largest |C| lands in [2^13, 2^14)
  __shared__ float s_red[kThreads / 64];
  __shared__ half4_t s_ah[8 * 64], s_al[8 * 64];  // A operands [T][lane], hi and lo parts
  __shared__ float s_norm[256];                    // |c 2^sc|^2, +inf past n_c
  __shared__ float s_seeded[kThreads / 64][256];   // per wave: s_norm 2^(s - sc) of a rescaled step
  int sc;
  {
    const int c = threadIdx.x;
    float m = 0.f;
    if (c < d.n_c) {
#pragma unroll
      for (int e = 0; e < DS; ++e) m = fmaxf(m, fabsf(cb[c * DS + e]));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) s_red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    sc = m > 0.f ? 14 - __builtin_amdgcn_frexp_expf(m) : 0;
    float n = INFINITY;
    if (c < d.n_c) {
      n = 0.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) {
        const float v = ldexpf(cb[c * DS + e], sc);
        n = fmaf(v, v, n);
      }
    }
    s_norm[c] = n;
    // entries (T, ln) for T = 2 (threadIdx / 64) + r
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int T = 2 * wave + r;
      const int cc = 32 * T + l32;
      half4_t ah, al;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float v = cc < d.n_c ? -2.f * ldexpf(cb[cc * DS + 4 * hi + u], sc) : 0.f;
        ah[u] = (_Float16)v;
        al[u] = (_Float16)(v - (float)ah[u]);
      }
      s_ah[T * 64 + lane] = ah;
      s_al[T * 64 + lane] = al;
    }
  }

  const int n_th = d.B * d.H * d.S;  // below 2^31 (the launcher checks)
  const int n_steps = (n_th + TPW - 1) / TPW;
  const int stride = (int)gridDim.x * WPB;
  // row 32 g + l32 of the step at token-head th0
  auto th_of = [&](int th0, int g) { return th0 + (32 * g + l32) / NSUB; };
  auto j_of = [&](int g) { return (32 * g + l32) % NSUB; };

  uint2 raw[2];
  float4 sv[2];
  auto load_rows = [&](int th0) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      int th = th_of(th0, g);
      th = th < n_th ? th : 0;
      raw[g] = *reinterpret_cast<const uint2*>(keys + (long long)th * D + j_of(g) * DS + 4 * hi);
      if (smooth) {
        const int bh = (int)fast_div((uint32_t)th, d.div_S);
        const int h = d.smooth_rows == 1 ? 0 : bh - (int)fast_div((uint32_t)bh, d.div_H) * d.H;
        sv[g] = *reinterpret_cast<const float4*>(smooth + h * D + j_of(g) * DS + 4 * hi);
      }
    }
  };

  int step = (int)blockIdx.x * WPB + wave;
  load_rows((step < n_steps ? step : 0) * TPW);
  __syncthreads();

  for (; step < n_steps; step += stride) {
    const int th0 = step * TPW;
    float x[2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const bool valid = th_of(th0, g) < n_th;
      const uint32_t w[2] = {raw[g].x, raw[g].y};
      const float svv[4] = {sv[g].x, sv[g].y, sv[g].z, sv[g].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint16_t b = (uint16_t)(w[u >> 1] >> (16 * (u & 1)));
        float v = valid ? __half2float(*reinterpret_cast<const __half*>(&b)) : 0.f;
        // x / s as x * rcp(s) (within 2 ulp of the quotient; such a
        // difference can only move a code at a near-tie)
        if (smooth) v = v * __builtin_amdgcn_rcpf(svv[u]);
        x[g][u] = v;
      }
    }
    float4 svc[2];  // this step's smooth factors, for the reconstruction
    if constexpr (MODE == 1) {
      svc[0] = sv[0];
      svc[1] = sv[1];
    }
    load_rows((step + stride < n_steps ? step + stride : step) * TPW);
    if (d.transform) wht_b8<D>(x, lane);

    // the step's scale: 2^sc unless that would leave the fp16 range
    float mx = 0.f;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) mx = fmaxf(mx, fabsf(x[g][u]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    int s = sc;
    const float* nrm = s_norm;  // accumulator seeds |c 2^sc|^2 2^(s - sc)
    if (ldexpf(mx, sc) >= 32768.f) {
      s = 14 - __builtin_amdgcn_frexp_expf(mx);
      // this wave's own seeds (its LDS accesses run in issue order, so the
      // reads below see them)
      float* w = s_seeded[wave];
      const float4 nv = *reinterpret_cast<const float4*>(s_norm + 4 * lane);
      const float f = ldexpf(1.f, s - sc);
      *reinterpret_cast<float4*>(w + 4 * lane) = make_float4(nv.x * f, nv.y * f, nv.z * f, nv.w * f);
      nrm = w;
    }
    half4_t bh[2], bl[2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float v = ldexpf(x[g][u], s);
        bh[g][u] = (_Float16)v;
        bl[g][u] = (_Float16)(v - (float)bh[g][u]);
      }

    struct TileIn {
      half4_t ah, al;
      float16_t n;
    };
    float best[2] = {INFINITY, INFINITY};
    int bi[2] = {0, 0}, bt[2] = {0, 0};  // offset in the tile, tile of the running minimum
    auto tile_in = [&](int T) {
      // re-read per stage (a compiler barrier keeps the 8 tiles' operands
      // from being hoisted out of the step loop into live registers)
      asm volatile("" ::: "memory");
      TileIn t;
      t.ah = s_ah[T * 64 + lane];
      t.al = s_al[T * 64 + lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 nv = *reinterpret_cast<const float4*>(nrm + 32 * T + 8 * q + 4 * hi);
        t.n[4 * q] = nv.x; t.n[4 * q + 1] = nv.y; t.n[4 * q + 2] = nv.z; t.n[4 * q + 3] = nv.w;
      }
      return t;
    };
    auto chains = [&](const TileIn& t, float16_t (&acc)[2]) {
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x8f16(t.ah, bh[0], t.n, 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x8f16(t.ah, bh[1], t.n, 0, 0, 0);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x8f16(t.al, bh[0], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x8f16(t.al, bh[1], acc[1], 0, 0, 0);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x8f16(t.ah, bl[0], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x8f16(t.ah, bl[1], acc[1], 0, 0, 0);
    };
    // candidates in increasing index order: offsets 8 (v / 4) + v mod 4 are
    // inline constants; the tile is recorded once per tile if it improved
    auto scan = [&](const float16_t (&r)[2], int T) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const float before = best[g];
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (r[g][v] < best[g]) { best[g] = r[g][v]; bi[g] = 8 * (v >> 2) + (v & 3); }
        if (best[g] < before) bt[g] = T;
      }
    };
    float16_t acc[2];
    chains(tile_in(0), acc);
    TileIn nxt_in = tile_in(1);
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      float16_t r[2] = {acc[0], acc[1]};
      if (T + 1 < 8) {
        chains(nxt_in, acc);
        if (T + 2 < 8) nxt_in = tile_in(T + 2);
      }
      scan(r, T);
      // Pin the stage in program order (IR passes otherwise regroup the
      // independent argmin chains across all tiles, keeping every tile's
      // accumulators live).
#pragma unroll
      for (int g = 0; g < 2; ++g)
        asm volatile("" : "+v"(best[g]), "+v"(bi[g]), "+v"(bt[g]), "+v"(acc[g]));
      __builtin_amdgcn_sched_barrier(0);
    }

    // merge lanes l and l ^ 32 (the two halves of every tile), lowest index on ties
    int idx[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float bv = best[g];
      int bx = 32 * bt[g] + bi[g] + 4 * hi;
      const float ov = __shfl_xor(bv, 32);
      const int ox = __shfl_xor(bx, 32);
      if (ov < bv || (ov == bv && ox < bx)) bx = ox;
      // (a row that never compares below +inf, e.g. NaN input, keeps a start index)
      idx[g] = min(bx, d.n_c - 1);
    }

    // lane l writes the code of row (g = l / 32, l mod 32)
    {
      const int code = hi ? idx[1] : idx[0];
      const int th = th_of(th0, hi);
      if (th < n_th) {
        const int bhh = (int)fast_div((uint32_t)th, d.div_S);
        const int t = th - bhh * d.S;
        const int off = d.use_row_offsets ? offs.v[fast_div((uint32_t)bhh, d.div_H)] : d.S_off;
        codes[((long long)bhh * d.S_cap + off + t) * NSUB + j_of(hi)] = (uint8_t)code;
      }
    }
    if constexpr (MODE == 1) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const float4 cv = *reinterpret_cast<const float4*>(cb + idx[g] * DS + 4 * hi);
        x[g][0] = cv.x; x[g][1] = cv.y; x[g][2] = cv.z; x[g][3] = cv.w;
      }
      if (d.transform) wht_b8<D>(x, lane);  // H is its own inverse
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int th = th_of(th0, g);
        if (th >= n_th) continue;
        float o[4] = {x[g][0], x[g][1], x[g][2], x[g][3]};
        if (smooth) {
          o[0] *= svc[g].x; o[1] *= svc[g].y; o[2] *= svc[g].z; o[3] *= svc[g].w;
        }
        const long long base = (long long)th * D + j_of(g) * DS + 4 * hi;
        if (d.recon_dtype == 1) {
          const __half2 a = __floats2half2_rn(o[0], o[1]), b = __floats2half2_rn(o[2], o[3]);
          uint2 u;
          u.x = *reinterpret_cast<const uint32_t*>(&a);
          u.y = *reinterpret_cast<const uint32_t*>(&b);
          *reinterpret_cast<uint2*>(reinterpret_cast<__half*>(recon) + base) = u;
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(recon) + base) =
              make_float4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  }
}

template <int D, int DS, int MODE>
void launch_mfma(const EncodeArgs& a, const Dims& d, const RowOffsets& o, hipStream_t st) {
  constexpr int NSUB = D / DS;
  // sub-vectors of 8 run the split-fp16 kernel, 4 and 16 the fp32 one
  void (*kern)(const __half*, const float*, const float*, uint8_t*, void*, Dims, RowOffsets);
  if constexpr (DS == 8) kern = pvq_f16_kernel<D, MODE>;
  else kern = pvq_mfma_kernel<D, DS, MODE>;
  // as many workgroups as are resident at once (one pass of waves over the
  // steps, no partial second round), from the kernel's own occupancy; cached
  // per device (any thread may launch: relaxed atomics, same value if raced)
  static std::atomic<int> resident[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) dev = 0;
  int res = resident[dev].load(std::memory_order_relaxed);
  if (res <= 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    res = per_cu * cus;
    resident[dev].store(res, std::memory_order_relaxed);
  }
  const long long n_th = (long long)a.B * a.H * a.S;
  const long long n_steps = (n_th + 64 / NSUB - 1) / (64 / NSUB);
  const long long want = (n_steps + kThreads / 64 - 1) / (kThreads / 64);
  const unsigned blocks = (unsigned)std::min(want, (long long)res);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), 0, st, a.keys, a.codebook, a.smooth,
                     a.codes, a.recon, d, o);
}

template <int D, int DS, int MODE, int CSPLIT>
void launch_one(const EncodeArgs& a, const Dims& d, const RowOffsets& o, hipStream_t st) {
  constexpr int NSUB = D / DS;
  constexpr int NT = threads_for<CSPLIT>();
  constexpr int TPB = (NT / 64 / CSPLIT) * (64 / NSUB);
  const long long n_th = (long long)a.B * a.H * a.S;
  const unsigned blocks = (unsigned)((n_th + TPB - 1) / TPB);
  hipLaunchKernelGGL((pvq_kernel<D, DS, MODE, CSPLIT>), dim3(blocks), dim3(NT), 0, st,
                     a.keys, a.codes_in, a.codebook, a.smooth, a.codes, a.recon, d, o);
}

// Stage a [D, D] matrix as the A operands of Y^T = M^T X^T on
// v_mfma_f32_32x32x8_f16: entry (kc, ct, lane) holds M[8 kc + 4 (lane / 32)
// + u][32 ct + lane mod 32], u < 4, scaled by 2^em so that the largest
// magnitude lands in [2^13, 2^14), split into fp16 hi and lo.  Every thread
// of the workgroup takes part; ends with a barrier.  Returns em.
template <int D, int NT>
__device__ __forceinline__ int stage_split_matrix(const float* __restrict__ rot, half4_t* s_mh,
                                                  half4_t* s_ml, float* s_red) {
  constexpr int NW = NT / 64, KC = D / 8, CT = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float m = 0.f;
  for (int i = threadIdx.x; i < D * D / 4; i += NT) {
    const float4 v = reinterpret_cast<const float4*>(rot)[i];
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) m = fmaxf(m, s_red[w]);
  const int em = m > 0.f ? 14 - __builtin_amdgcn_frexp_expf(m) : 0;
  for (int e = threadIdx.x; e < KC * CT * 64; e += NT) {
    const int kc = e / (CT * 64), ct = (e / 64) % CT, ln = e & 63;
    const int row = 8 * kc + 4 * (ln >> 5), col = 32 * ct + (ln & 31);
    half4_t h, l;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float v = ldexpf(rot[(row + u) * D + col], em);
      h[u] = (_Float16)v;
      l[u] = (_Float16)(v - (float)h[u]);
    }
    s_mh[e] = h;
    s_ml[e] = l;
  }
  __syncthreads();  // the matrix is staged; s_red may be reused
  return em;
}

// Dense rotation on the matrix cores, for the encode (sub-vectors of 8, 8-bit
// codes) and the transform-only mode: a wave takes 32 token-heads and forms
// Y^T = M^T X^T on v_mfma_f32_32x32x8_f16, A = M^T (32 output dims x 8 input
// dims per step, from LDS), B = X^T (8 input dims x 32 token-heads, the
// lane's own token-head), each operand split into fp16 high and low parts
// (three passes; the dropped lo.lo term is below 2^-22 of each product) and
// scaled by powers of two: M so that its largest entry lands in
// [2^13, 2^14), each token-head's x / s likewise.  The accumulator of output
// tile ct gives lane l the dims 32 ct + 8 q + 4 (l / 32) + u of token-head
// l mod 32: sub-vector j = 4 ct + q, elements 4 (l / 32) + u, which is the
// row layout of f16_nearest, so the search follows with no reshuffle.
template <int D, int MODE>
__global__ __launch_bounds__(512) void pvq_dense_mfma_kernel(
    const __half* __restrict__ keys, const float* __restrict__ cb, const float* __restrict__ smooth,
    const float* __restrict__ rot, uint8_t* __restrict__ codes, float* __restrict__ out, Dims d,
    RowOffsets offs) {
  constexpr int NW = 8, NT = NW * 64;
  constexpr int KC = D / 8, CT = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  __shared__ half4_t s_mh[KC * CT * 64], s_ml[KC * CT * 64];  // [kc][ct][lane]
  __shared__ float s_red[NW];
  __shared__ std::conditional_t<MODE == 0, F16Codebook, char> tab;
  __shared__ std::conditional_t<MODE == 0, float[NW][256], char> s_seeded;
  const int em = stage_split_matrix<D, NT>(rot, s_mh, s_ml, s_red);
  int sc = 0;
  if constexpr (MODE == 0) sc = f16_stage<NT>(cb, d.n_c, tab, s_red);
  else __syncthreads();

  const long long n_th = (long long)d.B * d.H * d.S;
  const long long n_tiles = (n_th + 31) / 32;
  for (long long tile = (long long)blockIdx.x * NW + wave; tile < n_tiles;
       tile += (long long)gridDim.x * NW) {
    const long long th = tile * 32 + l32;
    const bool valid = th < n_th;
    const long long thc = valid ? th : 0;
    const int bh = (int)(thc / d.S);
    const int h = bh % d.H;
    const __half* xr = keys + thc * D + 4 * hi;
    const float* sr = smooth ? smooth + (size_t)(d.smooth_rows == 1 ? 0 : h) * D + 4 * hi : nullptr;
    auto load = [&](int kc, float (&v)[4]) {
      const uint2 raw = *reinterpret_cast<const uint2*>(xr + 8 * kc);
      const float2 f0 = __half22float2(*reinterpret_cast<const __half2*>(&raw.x));
      const float2 f1 = __half22float2(*reinterpret_cast<const __half2*>(&raw.y));
      v[0] = f0.x; v[1] = f0.y; v[2] = f1.x; v[3] = f1.y;
      if (!valid) v[0] = v[1] = v[2] = v[3] = 0.f;
      if (sr) {
        const float4 sv = *reinterpret_cast<const float4*>(sr + 8 * kc);
        v[0] = v[0] / sv.x; v[1] = v[1] / sv.y; v[2] = v[2] / sv.z; v[3] = v[3] / sv.w;
      }
    };
    // this token-head's scale (both halves of the lane pair)
    float mx = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      float v[4];
      load(kc, v);
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const int ex = mx > 0.f ? 14 - __builtin_amdgcn_frexp_expf(mx) : 0;
    half4_t bh_[KC], bl_[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      float v[4];
      load(kc, v);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = ldexpf(v[u], ex);
        bh_[kc][u] = (_Float16)w;
        bl_[kc][u] = (_Float16)(w - (float)bh_[kc][u]);
      }
    }
    const int unscale = -(ex + em);
    const int t = (int)(thc - (long long)bh * d.S);
    const int b = bh / d.H;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float16_t acc = {};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const half4_t ah = s_mh[(kc * CT + ct) * 64 + lane], al = s_ml[(kc * CT + ct) * 64 + lane];
        acc = __builtin_amdgcn_mfma_f32_32x32x8f16(ah, bh_[kc], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x8f16(al, bh_[kc], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x8f16(ah, bl_[kc], acc, 0, 0, 0);
      }
      float y[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) y[v] = ldexpf(acc[v], unscale);
      if constexpr (MODE == 3) {
        if (valid) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(out + th * D + 32 * ct + 8 * q + 4 * hi) =
                make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]);
        }
        // one output tile at a time (the scheduler would otherwise keep every
        // tile's accumulators live)
        __builtin_amdgcn_sched_barrier(0);
      } else {
        const int off = d.use_row_offsets ? offs.v[b] : d.S_off;
#pragma unroll
        for (int qp = 0; qp < 2; ++qp) {
          const float x2[2][4] = {{y[8 * qp], y[8 * qp + 1], y[8 * qp + 2], y[8 * qp + 3]},
                                  {y[8 * qp + 4], y[8 * qp + 5], y[8 * qp + 6], y[8 * qp + 7]}};
          int idx[2];
          f16_nearest(x2, sc, tab, s_seeded[wave], d.n_c, idx);
          if (valid && !hi) {
            uint8_t* cp = codes + ((long long)bh * d.S_cap + off + t) * (D / 8) + 4 * ct + 2 * qp;
            cp[0] = (uint8_t)idx[0];
            cp[1] = (uint8_t)idx[1];
          }
        }
      }
    }
  }
}


// Decode with an explicit matrix (sub-vectors of 8) on the matrix cores, and
// the reconstruction half of a round trip: a wave takes 32 token-heads, reads
// each one's codes, gathers the centroid rows straight into the B operand
// layout from the staged search codebook (-2 C 2^sc as fp16 hi + lo, entry
// [code / 32][lane half][code mod 32]), and forms Y^T = (M^-1)^T X^T in three
// split-fp16 passes as the forward rotation; Y is unscaled by
// -2^-(sc + 1 + em), multiplied by s and stored (fp16 rounds to nearest).
// A code past n_c decodes as centroid n_c - 1, as on the per-lane path.
template <int D>
__global__ __launch_bounds__(512) void pvq_dense_mfma_decode_kernel(
    const uint8_t* __restrict__ codes_in, const float* __restrict__ cb, const float* __restrict__ smooth,
    const float* __restrict__ rot_inv, void* __restrict__ recon, Dims d, RowOffsets offs) {
  constexpr int NW = 8, NT = NW * 64;
  constexpr int KC = D / 8, CT = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  __shared__ half4_t s_mh[KC * CT * 64], s_ml[KC * CT * 64];  // [kc][ct][lane]
  __shared__ float s_red[NW];
  __shared__ F16Codebook tab;
  const int em = stage_split_matrix<D, NT>(rot_inv, s_mh, s_ml, s_red);
  const int sc = f16_stage<NT>(cb, d.n_c, tab, s_red);
  const int unscale = -(sc + 1 + em);
  const int row_bytes = d.code_bits == 4 ? KC / 2 : KC;

  const long long n_th = (long long)d.B * d.H * d.S;
  const long long n_tiles = (n_th + 31) / 32;
  for (long long tile = (long long)blockIdx.x * NW + wave; tile < n_tiles;
       tile += (long long)gridDim.x * NW) {
    const long long th = tile * 32 + l32;
    const bool valid = th < n_th;
    const long long thc = valid ? th : 0;
    const int bh = (int)(thc / d.S);
    const int h = bh % d.H;
    const int t = (int)(thc - (long long)bh * d.S);
    const int off = d.use_row_offsets ? offs.v[bh / d.H] : d.S_off;
    const uint8_t* cr = codes_in + ((long long)bh * d.S_cap + off + t) * row_bytes;
    half4_t bh_[KC], bl_[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      int c = d.code_bits == 4 ? ((cr[kc >> 1] >> (4 * (kc & 1))) & 15) : cr[kc];
      c = min(c, d.n_c - 1);
      const int e = (c >> 5) * 64 + hi * 32 + (c & 31);
      bh_[kc] = tab.ah[e];
      bl_[kc] = tab.al[e];
    }
    const float* sr = smooth ? smooth + (size_t)(d.smooth_rows == 1 ? 0 : h) * D + 4 * hi : nullptr;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float16_t acc = {};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const half4_t ah = s_mh[(kc * CT + ct) * 64 + lane], al = s_ml[(kc * CT + ct) * 64 + lane];
        acc = __builtin_amdgcn_mfma_f32_32x32x8f16(ah, bh_[kc], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x8f16(al, bh_[kc], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x8f16(ah, bl_[kc], acc, 0, 0, 0);
      }
      if (valid) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float y[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) y[u] = -ldexpf(acc[4 * q + u], unscale);
          if (sr) {
            const float4 sv = *reinterpret_cast<const float4*>(sr + 32 * ct + 8 * q);
            y[0] *= sv.x; y[1] *= sv.y; y[2] *= sv.z; y[3] *= sv.w;
          }
          const long long o = th * D + 32 * ct + 8 * q + 4 * hi;
          if (d.recon_dtype == 1)
            store_f16<4>(reinterpret_cast<__half*>(recon) + o, y);
          else
            store_f32<4>(reinterpret_cast<float*>(recon) + o, y);
        }
      }
      // one output tile at a time (the scheduler would otherwise keep every
      // tile's accumulators live)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

Dims make_dims(const EncodeArgs& a) {
  return Dims{a.B, a.H, a.S, a.n_c, a.smooth_rows, a.transform, a.S_cap, a.S_off,
              a.use_row_offsets, a.recon_dtype, make_fastdiv((uint32_t)a.S), make_fastdiv((uint32_t)a.H),
              a.code_bits};
}

// Fewer lanes than about four waves per CU (256 CUs): split the codebook
// over the waves of a workgroup instead of giving each its own token-heads,
// so short appends (one token per row) are not latency bound; below one wave
// per CU, 16 ways (16 waves per workgroup).
int codebook_split(const EncodeArgs& a) {
  const long long n_th = (long long)a.B * a.H * a.S;
  const long long lanes = n_th * (a.D / a.sub_dim);
  return lanes < 256LL * 64 ? 16 : (lanes < 256LL * 64 * 4 ? 4 : 1);
}

template <int D, int DS>
hipError_t launch_ds(const EncodeArgs& a, const RowOffsets* offs, int mode, hipStream_t st) {
  const long long n_th = (long long)a.B * a.H * a.S;
  if ((n_th + 3) / 4 > 0x7fffffffLL) return hipErrorInvalidValue;
  const Dims d = make_dims(a);
  RowOffsets o{};
  if (offs) o = *offs;
  if (a.transform == 2) {
    if constexpr (D <= 128) {
      // forward rotations on the matrix cores: the transform-only mode and
      // the encode of sub-vectors of 8 with 8-bit codes
      // one grid-stride pass of 512-thread workgroups, as many as are
      // resident at once, over tiles of 32 token-heads
      auto mfma_blocks = [&](const void* k) {
        int per_cu = 0, cus = 0, dev = 0;
        (void)hipGetDevice(&dev);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 512, 0) != hipSuccess || per_cu <= 0)
          per_cu = 1;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
          cus = 256;
        const long long tiles = (n_th + 31) / 32;
        const long long want = (tiles + 7) / 8;
        return (unsigned)std::max(1LL, std::min(want, (long long)per_cu * cus));
      };
      const bool fwd = mode == 3 || ((mode == 0 || mode == 1) && DS == 8 && a.code_bits == 8);
      if (fwd) {
        // the forward rotation (and the search): the transform-only mode,
        // and the encode of sub-vectors of 8 with 8-bit codes, also as the
        // first half of a round trip
        void (*mk)(const __half*, const float*, const float*, const float*, uint8_t*, float*, Dims,
                   RowOffsets) = mode == 3 ? pvq_dense_mfma_kernel<D, 3> : pvq_dense_mfma_kernel<D, 0>;
        hipLaunchKernelGGL(mk, dim3(mfma_blocks(reinterpret_cast<const void*>(mk))), dim3(512), 0, st,
                           a.keys, a.codebook, a.smooth, a.rot, a.codes, reinterpret_cast<float*>(a.recon),
                           d, o);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || mode != 1) return e;
      }
      if constexpr (DS == 8) {
        if (mode == 2 || (mode == 1 && fwd)) {
          // decode by M^-1: of the given codes, or (round trip) of the codes
          // the launch above wrote
          auto dk = pvq_dense_mfma_decode_kernel<D>;
          hipLaunchKernelGGL(dk, dim3(mfma_blocks(reinterpret_cast<const void*>(dk))), dim3(512), 0, st,
                             mode == 2 ? a.codes_in : a.codes, a.codebook, a.smooth, a.rot_inv, a.recon,
                             d, o);
          return hipGetLastError();
        }
      }
      // one grid-stride pass: as many workgroups as are resident at once;
      // the encode of sub-vectors of 8 (one matrix in LDS) runs 12 waves per
      // workgroup to keep the matrix-core search fed
      const int nmat = mode == 1 ? 2 : 1;
      const int nt = (DS == 8 && mode == 0) ? 768 : kThreads;
      const size_t lds = (size_t)(nmat * D * D + nt / 64 * 64 / (D / DS) * D) * sizeof(float);
      void (*kern)(const __half*, const uint8_t*, const float*, const float*, const float*,
                   const float*, uint8_t*, void*, Dims, RowOffsets);
      if (mode == 3) {
        if constexpr (DS == 8) kern = pvq_dense_kernel<D, DS, 3, kThreads>;
        else return hipErrorInvalidValue;
      } else if (mode == 0) {
        if constexpr (DS == 8) kern = pvq_dense_kernel<D, DS, 0, 768>;
        else kern = pvq_dense_kernel<D, DS, 0, kThreads>;
      } else {
        kern = mode == 1 ? pvq_dense_kernel<D, DS, 1, kThreads> : pvq_dense_kernel<D, DS, 2, kThreads>;
      }
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      int per_cu = 0, cus = 0, dev = 0;
      (void)hipGetDevice(&dev);
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, nt, lds) != hipSuccess ||
          per_cu <= 0)
        per_cu = 1;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          cus <= 0)
        cus = 256;
      const long long steps = (n_th + 64 / (D / DS) - 1) / (64 / (D / DS));
      const long long want = (steps + nt / 64 - 1) / (nt / 64);
      const unsigned blocks = (unsigned)std::max(1LL, std::min(want, (long long)per_cu * cus));
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(nt), lds, st, a.keys, a.codes_in, a.codebook,
                         a.smooth, a.rot, a.rot_inv, a.codes, a.recon, d, o);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (mode == 3) {  // forward transform only: one lane layout suffices
    if constexpr (DS == 8) {
      launch_one<D, DS, 3, 1>(a, d, o, st);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  const int split = codebook_split(a);
  // Enough sub-vectors to fill the chip: nearest centroid on the matrix cores
  // (8-bit codes; a 4-bit codebook has at most 16 centroids, a short search
  // for the per-lane kernel).
  if constexpr (DS % 4 == 0) {
    if (split == 1 && mode != 2 && a.code_bits == 8 && n_th < (1LL << 31)) {
      if (mode == 0) launch_mfma<D, DS, 0>(a, d, o, st);
      else launch_mfma<D, DS, 1>(a, d, o, st);
      return hipGetLastError();
    }
  }
  switch (mode) {
    case 0:
      if (split == 16) launch_one<D, DS, 0, 16>(a, d, o, st);
      else if (split == 4) launch_one<D, DS, 0, 4>(a, d, o, st);
      else launch_one<D, DS, 0, 1>(a, d, o, st);
      break;
    case 1:
      if (split == 16) launch_one<D, DS, 1, 16>(a, d, o, st);
      else if (split == 4) launch_one<D, DS, 1, 4>(a, d, o, st);
      else launch_one<D, DS, 1, 1>(a, d, o, st);
      break;
    default:
      launch_one<D, DS, 2, 1>(a, d, o, st);
      break;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const EncodeArgs& a, const RowOffsets* offs, int mode, hipStream_t st) {
  switch (a.sub_dim) {
    case 1: if constexpr (D / 1 <= 64) return launch_ds<D, 1>(a, offs, mode, st); break;
    case 2: if constexpr (D / 2 <= 64) return launch_ds<D, 2>(a, offs, mode, st); break;
    case 4: return launch_ds<D, 4>(a, offs, mode, st);
    case 8: return launch_ds<D, 8>(a, offs, mode, st);
    case 16: return launch_ds<D, 16>(a, offs, mode, st);
  }
  return hipErrorInvalidValue;
}

template <int D, int DSK, int DSV, int CSPLIT>
void launch_kv_fused(const EncodeArgs& k, const EncodeArgs& v, const RowOffsets& o, hipStream_t st) {
  constexpr int NT = threads_for<CSPLIT>();
  constexpr int TPBK = (NT / 64 / CSPLIT) * (64 / (D / DSK));
  constexpr int TPBV = (NT / 64 / CSPLIT) * (64 / (D / DSV));
  const long long n_th = (long long)k.B * k.H * k.S;
  const int kb = (int)((n_th + TPBK - 1) / TPBK), vb = (int)((n_th + TPBV - 1) / TPBV);
  hipLaunchKernelGGL((pvq_kv_kernel<D, DSK, DSV, CSPLIT>), dim3((unsigned)(kb + vb)), dim3(NT), 0, st,
                     k.keys, v.keys, k.codebook, v.codebook, k.smooth, k.codes, v.codes, make_dims(k),
                     make_dims(v), o, kb);
}

template <int D, int DSK, int DSV>
bool try_kv_fused(const EncodeArgs& k, const EncodeArgs& v, const RowOffsets& o, int split,
                  hipStream_t st) {
  if (k.sub_dim != DSK || v.sub_dim != DSV) return false;
  if (split == 16) {
    // the shortest appends: one token-head per workgroup
    const uint32_t n_th = (uint32_t)k.B * (uint32_t)k.H * (uint32_t)k.S;
    hipLaunchKernelGGL((pvq_short_kv_kernel<D, DSK, DSV>), dim3(2 * n_th), dim3(kThreads), 0, st, k.keys,
                       v.keys, k.codebook, v.codebook, k.smooth, k.codes, v.codes, make_dims(k),
                       make_dims(v), o, n_th);
  } else {
    launch_kv_fused<D, DSK, DSV, 4>(k, v, o, st);
  }
  return true;
}


// Lloyd assignment of fp32 sub-vectors of 8 on the matrix cores: the search
// of pvq_f16_kernel (|c|^2 - 2 c.x on v_mfma_f32_32x32x8_f16 with split-fp16
// operands and power-of-two scales, lowest index on ties; a rescaled step
// when values would leave the fp16 range) over vectors [N, 8], followed by
// the accumulation of the vector-ALU assignment kernel: per-centroid fp64
// sums and counts in LDS and the direct fp32 distance to the chosen
// centroid, written to the workgroup's row of partials.  Twelve waves per
// workgroup (three per SIMD), a wave step is 64 vectors.
constexpr int kKmWaves = 12;
__global__ __launch_bounds__(kKmWaves * 64) void kmeans_f16_kernel(
    const float* __restrict__ vecs, long long N, const float* __restrict__ cb, int n_c,
    double* __restrict__ partials, uint8_t* __restrict__ labels) {
  constexpr int DS = 8, W = DS + 1, NT = kKmWaves * 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  __shared__ double acc[256 * W + 1];
  __shared__ float s_red[kKmWaves];
  __shared__ F16Codebook tab;
  __shared__ float s_seeded[kKmWaves][256];
  const int slots = n_c * W + 1;
  for (int i = threadIdx.x; i < slots; i += NT) acc[i] = 0.0;
  const int sc = f16_stage<NT>(cb, n_c, tab, s_red);

  double inert = 0.0;
  const long long n_steps = (N + 63) / 64;
  for (long long step = (long long)blockIdx.x * kKmWaves + wave; step < n_steps;
       step += (long long)gridDim.x * kKmWaves) {
    // lane l holds elements 4 (l / 32) + u of vectors 64 step + 32 g + l mod 32
    float x[2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const long long row = step * 64 + 32 * g + l32;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row < N) v = *reinterpret_cast<const float4*>(vecs + row * DS + 4 * hi);
      x[g][0] = v.x; x[g][1] = v.y; x[g][2] = v.z; x[g][3] = v.w;
    }
    int idx[2];
    f16_nearest(x, sc, tab, s_seeded[wave], n_c, idx);
    // accumulate the two rows
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int ci = idx[g];
      const float4 cv = *reinterpret_cast<const float4*>(cb + ci * DS + 4 * hi);
      const float cvv[4] = {cv.x, cv.y, cv.z, cv.w};
      float d = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float df = x[g][u] - cvv[u];
        d = fmaf(df, df, d);
      }
      d += __shfl_xor(d, 32);
      const long long row = step * 64 + 32 * g + l32;
      if (row < N) {
        double* slot = acc + ci * W;
#pragma unroll
        for (int u = 0; u < 4; ++u) atomicAdd(slot + 4 * hi + u, (double)x[g][u]);
        if (!hi) {
          atomicAdd(slot + DS, 1.0);
          inert += (double)d;
          if (labels) labels[row] = (uint8_t)ci;
        }
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) inert += __shfl_xor(inert, m);
  if (lane == 0) atomicAdd(acc + n_c * W, inert);
  __syncthreads();
  double* row = partials + (size_t)blockIdx.x * slots;
  for (int i = threadIdx.x; i < slots; i += NT) row[i] = acc[i];
}

}  // namespace

hipError_t launch_kmeans_assign_f16(const float* vecs, long long N, const float* cb, int n_c,
                                    double* partials, int blocks, uint8_t* labels, hipStream_t st) {
  hipLaunchKernelGGL(kmeans_f16_kernel, dim3(blocks), dim3(kKmWaves * 64), 0, st, vecs, N, cb, n_c,
                     partials, labels);
  return hipGetLastError();
}

hipError_t launch_encode_kv(const EncodeArgs& k, const EncodeArgs& v, const RowOffsets* offs,
                            hipStream_t st) {
  // One launch when both halves are short appends on the split search with
  // the same split and a compiled (head dim, key, value sub_dim) triple;
  // otherwise the two encodes run one after the other.
  const int split = codebook_split(k);
  if (k.transform != 2 && split > 1 && split == codebook_split(v)) {
    RowOffsets o{};
    if (offs) o = *offs;
    bool done = false;
    if (k.D == 128) done = try_kv_fused<128, 8, 4>(k, v, o, split, st) || try_kv_fused<128, 4, 4>(k, v, o, split, st);
    else if (k.D == 64) done = try_kv_fused<64, 8, 4>(k, v, o, split, st) || try_kv_fused<64, 4, 4>(k, v, o, split, st);
    if (done) return hipGetLastError();
  }
  hipError_t e = launch_encode(k, offs, 0, st);
  if (e != hipSuccess) return e;
  return launch_encode(v, offs, 0, st);
}

hipError_t launch_encode(const EncodeArgs& a, const RowOffsets* offs, int mode, hipStream_t st) {
  switch (a.D) {
    case 32: return launch_d<32>(a, offs, mode, st);
    case 64: return launch_d<64>(a, offs, mode, st);
    case 128: return launch_d<128>(a, offs, mode, st);
    case 256: return launch_d<256>(a, offs, mode, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace vq
