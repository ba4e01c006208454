// Split-K attention from product-VQ codes with the value accumulation on
// MFMA (gfx950).
//
// Same method as the generic kernel ("Metal Kernels API" page, "Fused SDPA",
// metal_fused_sdpa; "veloxquant_mlx.cache.vecinfer_cache module" page,
// fused_sdpa): dual-transformed query, per-sub-vector query LUT, scores
// gathered by key codes, online softmax in base 2, values gathered from the
// value codebook by value codes.  This kernel covers value sub_dim 4 (one
// code -> 4 dims), D in {64, 128} and 8, 16 or 32 key sub-vectors.
//
// Per wave, keys stream in blocks of 64 (lane = key for the scores).  The
// value sum  out[r][4j+e] = sum_t p[r][t] C_v[vcode[t][j]][e]  runs on
// v_mfma_f32_4x4x4_16b_f16: block b = (token quad tq, subspace group sg) of
// the lane index l = 16 tq + 4 sg + n;  A_b = p[row][4 tokens of tq] (fp16,
// staged through 576 B of LDS per wave),  B_b[k][n] = C_v[code(t_k, j)][e]
// with j = 16 w + 4 sg + n for one (w, e) per instruction, so that the
// accumulation over tokens happens inside the MFMA and every lane keeps only
// 4 * (D / 64) float4 accumulators.  The lane's four codes (4 tokens, one
// subspace) come from one dword of codes per token and a 4x4 byte transpose
// across the lane quad (two DPP quad permutes + two v_perm).  Codebook rows
// are gathered as fp16 from LDS (8 bytes per code).
//
// Softmax rescaling is lazy: a block only rescales when some score exceeds
// the running max by more than 8 (log2 units), so p <= 256 (safe in fp16)
// and the common block needs no cross-lane reduction at all.
//
// Each workgroup writes the partial (m, l, acc[D]) of its rows; the merge
// kernel combines the splits with the log-sum-exp rule.
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kPstStride = 72;   // fp16 elements per staged P row (64 + pad)
constexpr float kLazyMargin = 8.f;
constexpr size_t kLdsBudget = 160 * 1024 - 256;  // headroom for static __shared__

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

struct MfmaLds {
  size_t lut, cv16, qt, pst, total_bytes;
};

// LDS layout in bytes.  The LUT and the fp16 value codebook always have 256
// entries (zero padded), so any code byte indexes a valid entry.
__host__ __device__ inline MfmaLds mfma_lds(int nsk, int R, int D) {
  MfmaLds L;
  size_t o = 0;
  size_t lut = (size_t)nsk * 256 * R * 4;
  // after the key loop the LUT area holds every lane's value partials
  const size_t red = (size_t)kWaves * 4 * D * R * 4;
  if (lut < red) lut = red;
  L.lut = o; o += (lut + 15) / 16 * 16;
  L.cv16 = o; o += 256 * 4 * 2;
  L.qt = o; o += (size_t)R * D * 4;
  L.pst = o; o += (size_t)kWaves * 4 * kPstStride * 2;
  L.total_bytes = (o + 15) / 16 * 16;
  return L;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <int CTRL>
__device__ __forceinline__ uint32_t quad_perm(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true);
}

template <int R>
__device__ __forceinline__ void lds_row(const float* e, float (&v)[R]) {
  if constexpr (R == 1) {
    v[0] = e[0];
  } else if constexpr (R == 2) {
    const float2 a = *reinterpret_cast<const float2*>(e);
    v[0] = a.x; v[1] = a.y;
  } else {
    const float4 a = *reinterpret_cast<const float4*>(e);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
}

template <int NSK>
struct KeyCodes {
  uint32_t w[NSK / 4];
};

template <int NSK>
__device__ __forceinline__ void load_key_codes(const uint8_t* p, KeyCodes<NSK>& k) {
  if constexpr (NSK % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NSK / 16; ++i) {
      const uint4 u = reinterpret_cast<const uint4*>(p)[i];
      k.w[4 * i] = u.x; k.w[4 * i + 1] = u.y; k.w[4 * i + 2] = u.z; k.w[4 * i + 3] = u.w;
    }
  } else {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    k.w[0] = u.x; k.w[1] = u.y;
  }
}

// Keeps a workgroup-uniform 64-bit value in SGPRs so that loads can use the
// scalar base + 32-bit vector offset form.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Byte rotation of the lane's NSK code bytes by 4 * rot_dw + rot_b:
// out byte k = in byte (k + 4 rot_dw + rot_b) mod NSK.
template <int NSK>
__device__ __forceinline__ void rotate_codes(const KeyCodes<NSK>& in, int rot_dw, int rot_b,
                                             uint32_t (&out)[NSK / 4]) {
  constexpr int NWD = NSK / 4;
  uint32_t dw[NWD];
#pragma unroll
  for (int d = 0; d < NWD; ++d) {
    uint32_t v = in.w[d];
#pragma unroll
    for (int s = 1; s < (NWD < 4 ? NWD : 4); ++s) v = (rot_dw == s) ? in.w[(d + s) % NWD] : v;
    dw[d] = v;
  }
#pragma unroll
  for (int d = 0; d < NWD; ++d)
    out[d] = __builtin_amdgcn_alignbyte(dw[(d + 1) % NWD], dw[d], (uint32_t)rot_b);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One split of one (batch row b, kv head g, row group rg): writes the
// partial (m, l, acc[D]) of each of the R rows to out_part, or, when `out`
// is given (the only split of its rows), the normalized fp16 rows to out
// with the merge's arithmetic (a / l, 0 for a row with no valid key).
template <int D, int R, int NSK>
__device__ __forceinline__ void split_body(
    const __half* __restrict__ q, const uint8_t* __restrict__ kcodes,
    const float* __restrict__ kcb, const float* __restrict__ smooth,
    const uint8_t* __restrict__ vcodes, const float* __restrict__ vcb,
    float* __restrict__ out_part, __half* __restrict__ out, const AttParams& p, int b, int g,
    int rg, int len, int s_lo, int s_hi) {
  constexpr int NSV = D / 4;     // value sub-vectors
  constexpr int NW = NSV / 16;   // 16-subspace groups per token
  constexpr int DK = D / NSK;    // key sub_dim
  constexpr int E = D / 64;      // query elements per lane in the transform
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const MfmaLds L = mfma_lds(NSK, R, D);
  float* lut = reinterpret_cast<float*>(smem_raw + L.lut);
  uint2* cv16 = reinterpret_cast<uint2*>(smem_raw + L.cv16);
  float* qt = reinterpret_cast<float*>(smem_raw + L.qt);
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform across the wave: keep it (and the block loop
  // it drives) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // valid keys of row r: [klo[r], khi[r]) within this split (empty for
  // padding rows); causal: t <= q_abs, window W: t > q_abs - W, with
  // q_abs = len - S_q + i (uniform values)
  int klo[R], khi[R];
  int lo_max = s_lo, hi_min = s_hi;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int gr = rg * R + r;
    const int qabs = len - p.Sq + (gr < p.rows ? gr % p.Sq : 0);
    int lo = s_lo, hi = s_hi;
    if (p.window > 0) lo = max(lo, qabs - p.window + 1);
    if (p.causal) hi = min(hi, qabs + 1);
    if (gr >= p.rows) hi = lo;
    klo[r] = lo;
    khi[r] = hi;
    lo_max = max(lo_max, lo);
    hi_min = min(hi_min, hi);
  }

  // ---- dual transform q~ = (q * s) . H, one wave per query row ---------
  const float* srow = smooth ? smooth + (size_t)(p.smooth_rows == 1 ? 0 : g) * D : nullptr;
  if (wave < R) {
    const int gr = rg * R + wave;
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = 0.f;
    if (gr < p.rows) {
      const int h = g * p.G + gr / p.Sq, i = gr % p.Sq;
      const __half* qr = q + (((size_t)b * p.Hq + h) * p.Sq + i) * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        x[e] = __half2float(qr[e]);
        if (srow) x[e] *= srow[lane * E + e];
      }
    }
    if (p.transform) {
#pragma unroll
      for (int hb = 1; hb < E; hb <<= 1)
#pragma unroll
        for (int e = 0; e < E; ++e)
          if ((e & hb) == 0) { const float a = x[e], c = x[e + hb]; x[e] = a + c; x[e + hb] = a - c; }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float y = __shfl_xor(x[e], m);
          x[e] = upper ? (y - x[e]) : (x[e] + y);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) qt[wave * D + lane * E + e] = x[e] * p.fold;
  } else if (wave < R + 4) {
    // fp16 value codebook, 256 rows, zero padded
    const int c = (wave - R) * 64 + lane;
    uint2 v = make_uint2(0u, 0u);
    if (c < p.n_c) {
      const float4 f = reinterpret_cast<const float4*>(vcb)[c];
      __half2 a = __floats2half2_rn(f.x, f.y), bb = __floats2half2_rn(f.z, f.w);
      v.x = *reinterpret_cast<uint32_t*>(&a);
      v.y = *reinterpret_cast<uint32_t*>(&bb);
    }
    cv16[c] = v;
  }
  __syncthreads();

  // ---- query LUT, layout [code][j][R] -----------------------------------
  // Entry (j, code) lives at ((code * NSK + j) * R) floats: its LDS bank
  // group depends on j only, so a pass of lanes that reads distinct j's is
  // conflict-free whatever the codes (see the rotated read order below).
  // Build: thread = (j, centroid c); its query slice stays in registers.
  {
    constexpr int CPI = kThreads / NSK;   // centroids per iteration
    const int j = tid % NSK;
    float qs[R][DK];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < DK; ++e) qs[r][e] = qt[r * D + j * DK + e];
    for (int c = tid / NSK; c < 256; c += CPI) {
      float acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.f;
      if (c < p.n_c) {
        const float* crow = kcb + (size_t)c * DK;
#pragma unroll
        for (int e = 0; e < DK; ++e) {
          const float ce = crow[e];
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r] = fmaf(qs[r][e], ce, acc[r]);
        }
      }
      float* dst = lut + ((size_t)c * NSK + j) * R;
      if constexpr (R == 4) {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      } else if constexpr (R == 2) {
        *reinterpret_cast<float2*>(dst) = make_float2(acc[0], acc[1]);
      } else {
        dst[0] = acc[0];
      }
    }
  }
  __syncthreads();

  // ---- main loop: 64-key blocks, interleaved over the waves ---------------
  const int tq = lane >> 4, sg = (lane >> 2) & 3, nn = lane & 3;
  const uint32_t sel1 = nn < 2 ? 0x05040100u : 0x03020706u;
  const uint32_t sel2 = (nn & 1) ? 0x03070105u : 0x06020400u;
  _Float16* pw = reinterpret_cast<_Float16*>(smem_raw + L.pst) + wave * 4 * kPstStride;
  const uint64_t row0 = uniform_u64(((uint64_t)b * p.Hkv + g) * (uint64_t)p.S_cap);
  const uint8_t* kbase = kcodes + row0 * NSK;
  const uint8_t* vbase = vcodes + row0 * NSV;

  float m[R], l[R];
#pragma unroll
  for (int r = 0; r < R; ++r) { m[r] = -INFINITY; l[r] = 0.f; }
  float4_t acc[NW][4];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[w][e] = float4_t{0.f, 0.f, 0.f, 0.f};

  // rotated visiting order of the key sub-vectors: lane rotation rot, byte
  // offsets of each visited j inside a LUT row
  constexpr int NROT = NSK < 16 ? NSK : 16;
  const int rot = lane & (NROT - 1);
  const int rot_dw = rot >> 2, rot_b = rot & 3;
  uint32_t jterm[NSK];
#pragma unroll
  for (int k = 0; k < NSK; ++k) jterm[k] = (uint32_t)(((k + rot) % NSK) * R * 4);

  const int n_blk = (s_hi - s_lo + 63) / 64;
  KeyCodes<NSK> kr, krn;
  uint32_t vr[4][NW];

  // 32-bit byte offsets from the (uniform) row bases keep the address math
  // in one VALU op per load.  Key codes of the next block are fetched at the
  // top of an iteration, value codes at its end (they are consumed second).
  auto load_keys = [&](int blk, KeyCodes<NSK>& k) {
    const uint32_t tk = (uint32_t)min(s_lo + blk * 64 + lane, s_hi - 1);
    load_key_codes<NSK>(kbase + tk * (uint32_t)NSK, k);
  };
  auto load_values = [&](int blk) {
    const int t0 = s_lo + blk * 64;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const uint32_t tv = (uint32_t)min(t0 + 16 * gq + 4 * tq + nn, s_hi - 1);
      const uint32_t* vp = reinterpret_cast<const uint32_t*>(vbase + tv * (uint32_t)NSV);
#pragma unroll
      for (int w = 0; w < NW; ++w) vr[gq][w] = vp[4 * w + sg];
    }
  };

  int blk = wave;
  if (blk < n_blk) { load_keys(blk, kr); load_values(blk); }
  for (; blk < n_blk; blk += kWaves) {
    const bool more = blk + kWaves < n_blk;
    if (more) load_keys(blk + kWaves, krn);

    // scores: sum of LUT entries over the key sub-vectors, visited in the
    // lane's rotated order j = (k + rot) mod NSK (rotated code bytes)
    const int t = s_lo + blk * 64 + lane;
    uint32_t rc[NSK / 4];
    rotate_codes<NSK>(kr, rot_dw, rot_b, rc);
    float sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) sc[r] = 0.f;
#pragma unroll
    for (int jw = 0; jw < NSK / 4; ++jw) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t code = (rc[jw] >> (8 * k)) & 0xff;
        float v[R];
        lds_row<R>(reinterpret_cast<const float*>(
                       reinterpret_cast<const unsigned char*>(lut) +
                       (code * (uint32_t)(NSK * R * 4) + jterm[jw * 4 + k])), v);
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r] += v[r];
      }
      // at most 4 LUT rows in flight: bounds the register footprint
      __builtin_amdgcn_sched_barrier(0);
    }
    const int t0 = s_lo + blk * 64;
    if (t0 < lo_max || t0 + 64 > hi_min) {   // block straddles a row's range
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (t < klo[r] || t >= khi[r]) sc[r] = -INFINITY;
    }
    bool need = false;
#pragma unroll
    for (int r = 0; r < R; ++r) need = need || (sc[r] > m[r] + kLazyMargin);
    if (__any(need)) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float M = wave_max(sc[r]);
        if (M > m[r]) {
          const float a = (m[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[r] - M);
          m[r] = M;
          l[r] *= a;
#pragma unroll
          for (int w = 0; w < NW; ++w)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[w][e][r] *= a;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float pr = 0.f;
      if (r < R) {
        pr = (sc[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[r] - m[r]);
        l[r] += pr;
      }
      pw[r * kPstStride + lane] = (_Float16)pr;
    }
    wave_sync_lds();

    // values: 4 groups of 16 keys, 4 * NW MFMAs each
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      half4_t A = *reinterpret_cast<const half4_t*>(pw + nn * kPstStride + 16 * gq + 4 * tq);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint32_t X = vr[gq][w];
        const uint32_t Z = __builtin_amdgcn_perm(quad_perm<0x4E>(X), X, sel1);
        const uint32_t Y = __builtin_amdgcn_perm(quad_perm<0xB1>(Z), Z, sel2);
        const uint2 R0 = cv16[Y & 0xff];
        const uint2 R1 = cv16[(Y >> 8) & 0xff];
        const uint2 R2 = cv16[(Y >> 16) & 0xff];
        const uint2 R3 = cv16[Y >> 24];
        uint2 B0, B1, B2, B3;
        B0.x = __builtin_amdgcn_perm(R1.x, R0.x, 0x05040100u);
        B0.y = __builtin_amdgcn_perm(R3.x, R2.x, 0x05040100u);
        B1.x = __builtin_amdgcn_perm(R1.x, R0.x, 0x07060302u);
        B1.y = __builtin_amdgcn_perm(R3.x, R2.x, 0x07060302u);
        B2.x = __builtin_amdgcn_perm(R1.y, R0.y, 0x05040100u);
        B2.y = __builtin_amdgcn_perm(R3.y, R2.y, 0x05040100u);
        B3.x = __builtin_amdgcn_perm(R1.y, R0.y, 0x07060302u);
        B3.y = __builtin_amdgcn_perm(R3.y, R2.y, 0x07060302u);
        acc[w][0] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, __builtin_bit_cast(half4_t, B0), acc[w][0], 0, 0, 0);
        acc[w][1] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, __builtin_bit_cast(half4_t, B1), acc[w][1], 0, 0, 0);
        acc[w][2] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, __builtin_bit_cast(half4_t, B2), acc[w][2], 0, 0, 0);
        acc[w][3] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, __builtin_bit_cast(half4_t, B3), acc[w][3], 0, 0, 0);
      }
      // one 16-key group at a time: bounds the gathered rows held in registers
      __builtin_amdgcn_sched_barrier(0);
    }
    wave_sync_lds();

    if (more) {
      load_values(blk + kWaves);
      kr = krn;
    }
  }

  // ---- combine lanes and waves through LDS ----------------------------------
  // red[wave][tq][d][r]: this lane's accumulators cover dims
  // 4 (16 w + 4 sg + n) + e of rows r, summed over its token quad tq.
  float* red = reinterpret_cast<float*>(smem_raw + L.lut);
  float* wm = reinterpret_cast<float*>(smem_raw + L.pst);  // [kWaves][R]
  float* wl = wm + kWaves * R;                             // [kWaves][R]
  float lsum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float v = l[r];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    lsum[r] = v;
  }
  __syncthreads();   // every wave is done with the LUT and the P staging
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float* dst = red + (((size_t)wave * 4 + tq) * D + 4 * (16 * w + 4 * sg + nn) + e) * R;
      if constexpr (R == 4) {
        *reinterpret_cast<float4_t*>(dst) = acc[w][e];
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) dst[r] = acc[w][e][r];
      }
    }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) { wm[wave * R + r] = m[r]; wl[wave * R + r] = lsum[r]; }
  }
  __syncthreads();
  for (int idx = tid; idx < R * D; idx += kThreads) {
    const int r = idx / D, d = idx % D;
    if (rg * R + r >= p.rows) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w * R + r]);
    float a = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = wm[w * R + r];
      const float om = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      float sw = 0.f;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) sw += red[(((size_t)w * 4 + t4) * D + d) * R + r];
      a += om * sw;
      lt += om * wl[w * R + r];
    }
    if (out) {
      const int gr = rg * R + r;  // query row of the kv head: (head hl, position i)
      const int hl = gr / p.Sq, i = gr - hl * p.Sq;
      out[((size_t)(b * p.Hq + g * p.G + hl) * p.Sq + i) * D + d] =
          __float2half_rn(lt > 0.f ? a / lt : 0.f);
      continue;
    }
    out_part[r * (D + 2) + 2 + d] = a;
    if (d == 0) {
      out_part[r * (D + 2)] = M;
      out_part[r * (D + 2) + 1] = lt;
    }
  }
}

template <int D, int R, int NSK>
__global__ __launch_bounds__(kThreads, 4) void attend_mfma_kernel(
    const __half* __restrict__ q, const uint8_t* __restrict__ kcodes,
    const float* __restrict__ kcb, const float* __restrict__ smooth,
    const uint8_t* __restrict__ vcodes, const float* __restrict__ vcb,
    const int32_t* __restrict__ kv_lens, float* __restrict__ part, __half* __restrict__ out,
    AttParams p) {
  const int unit = blockIdx.x;  // b * Hkv + g
  const int rg = blockIdx.y;
  const int s = blockIdx.z;
  const int b = unit / p.Hkv, g = unit % p.Hkv;
  int len = kv_lens ? kv_lens[b] : p.S_cap;
  len = min(max(len, 0), p.S_cap);
  const int lo_all = p.window > 0 ? max(0, len - p.Sq - p.window + 1) : 0;
  const int s_lo = lo_all + s * p.split_tokens;
  const int s_hi = min(s_lo + p.split_tokens, len);
  float* out_part = part + (((size_t)unit * p.n_rgroups + rg) * p.n_split + s) * R * (D + 2);
  // a single split writes the output rows itself (no merge launch)
  __half* const direct = p.n_split == 1 ? out : nullptr;
  if (s_lo >= s_hi) {
    if (direct) {
      // no valid key for these rows: zeros
      for (int idx = threadIdx.x; idx < R * D; idx += kThreads) {
        const int r = idx / D, d = idx % D, gr = rg * R + r;
        if (gr >= p.rows) continue;
        const int hl = gr / p.Sq, i = gr - hl * p.Sq;
        direct[((size_t)(b * p.Hq + g * p.G + hl) * p.Sq + i) * D + d] = __float2half_rn(0.f);
      }
      return;
    }
    // nothing to attend in this split: an empty partial
    if (threadIdx.x < R) {
      out_part[threadIdx.x * (D + 2)] = -INFINITY;
      out_part[threadIdx.x * (D + 2) + 1] = 0.f;
    }
    return;
  }
  split_body<D, R, NSK>(q, kcodes, kcb, smooth, vcodes, vcb, out_part, direct, p, b, g, rg, len,
                        s_lo, s_hi);
}

template <int D, int R, int NSK>
hipError_t launch3(const AttendArgs& a, const AttParams& p, size_t lds, hipStream_t st) {
  auto k = attend_mfma_kernel<D, R, NSK>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid(a.B * a.Hkv, p.n_rgroups, p.n_split);
  hipLaunchKernelGGL(k, grid, dim3(kThreads), lds, st, a.q, a.k_codes, a.k_codebook, a.smooth,
                     a.v_codes, a.v_codebook, a.kv_lens, a.partials, a.out, p);
  return hipGetLastError();
}

template <int D, int R>
hipError_t launch2(const AttendArgs& a, const AttParams& p, size_t lds, hipStream_t st) {
  switch (p.nsk) {
    case 8: return launch3<D, R, 8>(a, p, lds, st);
    case 16: return launch3<D, R, 16>(a, p, lds, st);
    case 32: return launch3<D, R, 32>(a, p, lds, st);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch1(const AttendArgs& a, const AttParams& p, size_t lds, hipStream_t st) {
  switch (p.R) {
    case 1: return launch2<D, 1>(a, p, lds, st);
    case 2: return launch2<D, 2>(a, p, lds, st);
    case 4: return launch2<D, 4>(a, p, lds, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool attend_mfma_plan(int D, int dv, int nsk, int rows, int* R, size_t* lds_bytes) {
  if (!(D == 64 || D == 128) || dv != 4 || !(nsk == 8 || nsk == 16 || nsk == 32)) return false;
  if (D / nsk > 16) return false;
  int r = 1;
  while (r < rows && r < 4) r <<= 1;
  const size_t bytes = mfma_lds(nsk, r, D).total_bytes;
  if (bytes > kLdsBudget) return false;
  *R = r;
  *lds_bytes = bytes;
  return true;
}

hipError_t launch_attend_mfma(const AttendArgs& a, const AttParams& p, size_t lds, hipStream_t st) {
  hipError_t e = hipErrorInvalidValue;
  switch (a.D) {
    case 64: e = launch1<64>(a, p, lds, st); break;
    case 128: e = launch1<128>(a, p, lds, st); break;
  }
  if (e != hipSuccess) return e;
  if (p.n_split == 1) return hipSuccess;  // the kernel wrote the rows
  // The splits are combined by a second, small kernel.  (Merging in the last
  // workgroup of each unit needs device-scope release/acquire fences, which
  // on this part write back / invalidate the L2 and cost far more than the
  // extra launch.)
  return launch_attend_merge(a, p, st);
}

}  // namespace vq
