// Many-query attention from product-VQ codes (gfx950): the prefill chunk,
// where every kv head has at least 64 query rows.  Head dim 128, key sub_dim
// 8, value sub_dim 4.
//
// Same method as the decode kernels ("Metal Kernels API" page, "Fused SDPA",
// metal_fused_sdpa; "veloxquant_mlx.cache.vecinfer_cache module" page,
// fused_sdpa): dual-transformed query q~ = (q * s) . H, scores q~ . C_k[codes]
// (equal to q . K_hat), online softmax in base 2 over split chunks, values
// from the value codebook.  With many query rows per key, each decoded key
// or value row is reused by 256 rows, so both products run as dense MFMA
// tiles (v_mfma_f32_16x16x32_f16):
//
//   workgroup  = (batch row b, kv head g, tile of 256 query rows, key split);
//                8 waves x 32 rows; keys stream in tiles of 64.
//   S^T        = K~ Q~^T per wave: A = key rows (M = 16 keys, K = 32 dims),
//                gathered straight from an fp16 copy of the key codebook in
//                LDS by the key codes (no decoded key tile), B = the wave's
//                query rows, held in registers for the whole kernel.  Both
//                are fp16 pairs (hi + lo, about 22 significant bits), and
//                each score is three passes (lo.hi + hi.lo + hi.hi): with
//                scores of tens of log2 units, one fp16 pass would perturb
//                the softmax weights by ~1e-3.
//   softmax    lazy online softmax per row (base 2, the running max moves
//                only when a tile exceeds it by more than 8); p rounds to
//                fp16 (nearest even) and the denominator sums the rounded
//                values, so the weights applied are exactly normalized.
//   O         += P V: A = p taken straight from the score registers (the
//                K slots of a lane are the keys its score tile holds), B =
//                V^T, decoded once per key tile by the whole workgroup into
//                an LDS tile [dim][key] whose key axis is permuted to match
//                those slots (a 4 x 4 byte transpose of the value codes
//                across each lane quad, then a 4 x 4 half transpose of the
//                gathered value rows).  Two V^T buffers alternate between
//                key tiles, so one barrier per tile (the tile's V^T is
//                complete) suffices: the buffer a tile writes was last read
//                two tiles before, ahead of the previous tile's barrier.
//
// Each workgroup writes (m, l, acc[128]) per query row and split; the split
// merge kernel combines them.
#include "vq_internal.h"

#include <algorithm>

namespace vq {
namespace {

constexpr int tW = 8;
constexpr int tThreads = tW * 64;
constexpr int tD = 128;
constexpr int tRT = tW * 32;  // query rows per workgroup
constexpr int tKT = 64;       // keys per tile
// The 16 lanes that one b128 LDS read serves together need 16 distinct bank
// quads (64 banks of 4 bytes): both parts of the key codebook have 16
// replicas and lane l reads replica l mod 16, so gathers by any codes are
// conflict-free.
constexpr uint32_t tKTab = 0;       // key codebook hi [256][16 replicas][8 fp16] 64 KiB
constexpr uint32_t tKLo = 65536;    // key codebook lo [256][8 replicas][8 fp16] 32 KiB
constexpr uint32_t tVTab = 98304;   // value codebook  [256][4 replicas][4 fp16]   8 KiB
constexpr uint32_t tVT = 106496;    // V^T tiles       [2][128 dims][72 fp16]     36 KiB
constexpr uint32_t tRowB = 144;     // bytes per V^T row (64 fp16 + pad)
constexpr uint32_t tAl = tVT + 2 * tD * tRowB;      // per-wave row rescale factors
constexpr uint32_t tLdsBytes = tAl + tW * 32 * 4;
static_assert(tLdsBytes <= 160 * 1024, "LDS budget");
constexpr float tLazyMargin = 8.f;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) uint8_t lds_byte;
template <typename T>
__device__ __forceinline__ T lds_ld(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(
      reinterpret_cast<const lds_byte*>((size_t)addr));
}
template <typename T>
__device__ __forceinline__ void lds_st(uint32_t addr, T v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(reinterpret_cast<lds_byte*>((size_t)addr)) = v;
}

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
  const __half2 h = __floats2half2_rn(a, b);
  return *reinterpret_cast<const uint32_t*>(&h);
}

template <int CTRL>
__device__ __forceinline__ uint32_t quad_perm(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Valid key range [lo, hi) of query position i in a row of len keys.
__device__ __forceinline__ void pos_range(const TileParams& p, int len, int i, int& lo, int& hi) {
  const int qa = len - p.Sq + i;
  int h = p.causal ? (qa + 1 < len ? qa + 1 : len) : len;
  int l = p.window > 0 ? qa - p.window + 1 : 0;
  h = h > 0 ? h : 0;
  l = l > 0 ? l : 0;
  lo = l;
  hi = h > l ? h : l;
}

__global__ __launch_bounds__(tThreads, 1) void attend_tile_kernel(
    const __half* __restrict__ q, const uint8_t* __restrict__ k_codes,
    const float* __restrict__ k_codebook, const float* __restrict__ smooth,
    const uint8_t* __restrict__ v_codes, const float* __restrict__ v_codebook,
    const int32_t* __restrict__ kv_lens, float* __restrict__ part, TileParams p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = blockIdx.x % p.n_rt;
  const int bg = blockIdx.x / p.n_rt;
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;
  const int split = blockIdx.y;
  int len = p.S_cap;
  if (kv_lens) {
    const int v = kv_lens[b];
    len = v < 0 ? 0 : (v > p.S_cap ? p.S_cap : v);
  }

  // ---- codebooks into LDS (fp16, replicated across banks) -----------------
  // keys as an fp16 pair: hi = fp16(c), lo = fp16(c - hi)
  {
    const int code = tid >> 1, half = tid & 1;  // two threads per code
    float kf[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (code < p.n_c) {
      const float4 a = reinterpret_cast<const float4*>(k_codebook)[2 * code];
      const float4 c = reinterpret_cast<const float4*>(k_codebook)[2 * code + 1];
      kf[0] = a.x; kf[1] = a.y; kf[2] = a.z; kf[3] = a.w;
      kf[4] = c.x; kf[5] = c.y; kf[6] = c.z; kf[7] = c.w;
      v = reinterpret_cast<const float4*>(v_codebook)[code];
    }
    half8_t hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = (_Float16)kf[e];
      lo[e] = (_Float16)(kf[e] - (float)hi[e]);
    }
    const u32x2_t hv = {pack_half2(v.x, v.y), pack_half2(v.z, v.w)};
#pragma unroll
    for (int r = 4 * half; r < 4 * half + 4; ++r) {
      lds_st<half8_t>(tKTab + code * 256 + r * 16, hi);
      lds_st<half8_t>(tKTab + code * 256 + (r + 8) * 16, hi);
      lds_st<half8_t>(tKLo + code * 128 + r * 16, lo);
    }
#pragma unroll
    for (int r = 2 * half; r < 2 * half + 2; ++r) lds_st<u32x2_t>(tVTab + code * 32 + r * 8, hv);
  }

  // ---- key range of this workgroup: union over its rows, then the split ---
  const int gr0 = rt * tRT;
  const int grl = min(p.GS, gr0 + tRT) - 1;
  int i_lo = gr0 % p.Sq, i_hi = grl % p.Sq;
  if (gr0 / p.Sq != grl / p.Sq) { i_lo = 0; i_hi = p.Sq - 1; }  // spans two heads
  int lo, hi, dummy;
  pos_range(p, len, i_lo, lo, dummy);
  pos_range(p, len, i_hi, dummy, hi);
  const int range = hi > lo ? hi - lo : 0;
  const int cs = ((range + p.n_split - 1) / p.n_split + tKT - 1) / tKT * tKT;
  const int s_lo = lo + split * cs;
  const int s_hi = min(hi, s_lo + cs);

  // ---- the wave's 32 query rows: q~ as the B operand of S^T ----------------
  // lane (n = lane % 16, kg = lane / 16) holds, for row tile nt (0, 1), row
  // 32 wave + 16 nt + n and dims 32 c + 8 kg + e (c = 0..3, e = 0..7).
  const int n16 = lane & 15, kg = lane >> 4;
  half8_t qb[2][4], ql[2][4];  // q~ = qb + ql (fp16 pair: about 22 significant bits)
  int rlo[2], rhi[2];
  bool rvalid[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int gr = gr0 + 32 * wave + 16 * nt + n16;
    rvalid[nt] = gr < p.GS;
    const int grc = rvalid[nt] ? gr : p.GS - 1;
    const int hl = grc / p.Sq, ip = grc % p.Sq;
    pos_range(p, len, ip, rlo[nt], rhi[nt]);
    rlo[nt] = max(rlo[nt], s_lo);
    rhi[nt] = min(rhi[nt], s_hi);
    // rows past the last query row are computed unmasked and never written
    if (!rvalid[nt]) { rlo[nt] = s_lo; rhi[nt] = s_hi; }
    const __half* qp = q + ((size_t)(b * p.Hq + g * p.G + hl) * p.Sq + ip) * tD;
    float x[4][8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 w = *reinterpret_cast<const uint4*>(qp + 32 * c + 8 * kg);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 f = __half22float2(*reinterpret_cast<const __half2*>(&ww[k]));
        x[c][2 * k] = f.x;
        x[c][2 * k + 1] = f.y;
      }
    }
    if (smooth) {
      const float* sp = smooth + (p.smooth_rows == 1 ? 0 : g) * tD;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 s0 = *reinterpret_cast<const float4*>(sp + 32 * c + 8 * kg);
        const float4 s1 = *reinterpret_cast<const float4*>(sp + 32 * c + 8 * kg + 4);
        x[c][0] *= s0.x; x[c][1] *= s0.y; x[c][2] *= s0.z; x[c][3] *= s0.w;
        x[c][4] *= s1.x; x[c][5] *= s1.y; x[c][6] *= s1.z; x[c][7] *= s1.w;
      }
    }
    if (p.transform) {
      // in-register dim bits 0..2 (e) and 5..6 (c); dim bits 3..4 are lane bits 4..5
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (e & m) continue;
            const float u = x[c][e], w = x[c][e + m];
            x[c][e] = u + w;
            x[c][e + m] = u - w;
          }
      }
#pragma unroll
      for (int m = 1; m < 4; m <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c & m) continue;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float u = x[c][e], w = x[c + m][e];
            x[c][e] = u + w;
            x[c + m][e] = u - w;
          }
        }
      }
#pragma unroll
      for (int m = 16; m < 64; m <<= 1) {
        const float sg = (lane & m) ? -1.f : 1.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) x[c][e] = fmaf(sg, x[c][e], __shfl_xor(x[c][e], m));
      }
    }
    const float f = rvalid[nt] ? p.fold : 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = x[c][e] * f;
        qb[nt][c][e] = (_Float16)v;
        ql[nt][c][e] = (_Float16)(v - (float)qb[nt][c][e]);
      }
  }
  int full_lo = max(rlo[0], rlo[1]), full_hi = min(rhi[0], rhi[1]);
  // workgroup-uniform fast-path bounds: every valid row of the wave covers the tile
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    full_lo = max(full_lo, __shfl_xor(full_lo, o));
    full_hi = min(full_hi, __shfl_xor(full_hi, o));
  }

  // ---- per-lane constants ---------------------------------------------------
  const uint32_t kbase = tKTab + (uint32_t)(lane & 15) * 16u;    // key hi replica (256 B per code)
  const uint32_t kbase_lo = tKLo + (uint32_t)(lane & 7) * 16u;   // key lo replica (128 B per code)
  const uint32_t vtab = tVTab + (uint32_t)(lane & 3) * 8u;        // value replica
  // V^T decode task: lane quad (u = tid % 4) = keys 4 tq .. 4 tq + 3 x subs 4 sm .. 4 sm + 3,
  // quad tid / 4 = 16 sm + tq, so that the 32 lanes of each 8-byte V^T write
  // (4 dims x 8 key quads) land on distinct bank pairs
  const int qu = tid & 3;
  const uint32_t tsel1 = qu < 2 ? 0x05040100u : 0x03020706u;
  const uint32_t tsel2 = (qu & 1) ? 0x03070105u : 0x06020400u;

  float m_run[2] = {-INFINITY, -INFINITY}, th[2] = {-INFINITY, -INFINITY}, mref[2] = {0.f, 0.f};
  float lsum[2] = {0.f, 0.f};
  float4_t oacc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const size_t row_tok = (size_t)bg * p.S_cap;
  const uint8_t* const kc_row = k_codes + row_tok * 16;
  const uint8_t* const vc_row = v_codes + row_tok * 32;
  const int tmax = p.S_cap - 1;

  auto load_codes = [&](int tb, uint4 (&kc)[4], uint32_t (&vc)[1]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      kc[mt] = *reinterpret_cast<const uint4*>(kc_row + (size_t)min(tb + 16 * mt + n16, tmax) * 16);
    const int quad = tid >> 2;  // 128 quads: (key quad tq, sub group sm)
    const int tq = quad & 15, sm = quad >> 4;
    vc[0] = *reinterpret_cast<const uint32_t*>(vc_row + (size_t)min(tb + 4 * tq + qu, tmax) * 32 + 4 * sm);
  };

  uint4 kc[4];
  uint32_t vc[1];

  // one key tile; the next tile's codes are requested once this one's have
  // been consumed (after the scores), so they arrive during softmax and P V
  auto tile = [&](int tb, uint32_t vtb) {
    // ---- V^T tile of this key tile, decoded by the whole workgroup --------
    // (two buffers: the one written here was last read two tiles ago, before
    // the previous tile's barrier)
#pragma unroll
    for (int j = 0; j < 1; ++j) {
      const int quad = tid >> 2;
      const int tq = quad & 15, sm = quad >> 4;
      const uint32_t X = vc[j];
      const uint32_t Z = __builtin_amdgcn_perm(quad_perm<0x4E>(X), X, tsel1);
      const uint32_t Y = __builtin_amdgcn_perm(quad_perm<0xB1>(Z), Z, tsel2);
      // Y: codes of sub 4 sm + qu for keys 4 tq + 0..3
      const u32x2_t R0 = lds_ld<u32x2_t>(vtab + ((Y & 0xffu) << 5));
      const u32x2_t R1 = lds_ld<u32x2_t>(vtab + (((Y >> 8) & 0xffu) << 5));
      const u32x2_t R2 = lds_ld<u32x2_t>(vtab + (((Y >> 16) & 0xffu) << 5));
      const u32x2_t R3 = lds_ld<u32x2_t>(vtab + ((Y >> 24) << 5));
      const uint32_t dim0 = 4 * (4 * sm + qu);
      // keys 4 tq .. 4 tq + 3 (tq = 8 c2 + 4 h + kg) go to positions
      // 32 c2 + 8 kg + 4 h .. + 3 of the tile's key axis: the order in which
      // the P V operand slots take the weights straight from the score
      // registers
      const uint32_t kpos = 32u * (uint32_t)(tq >> 3) + 8u * (uint32_t)(tq & 3) + 4u * (uint32_t)((tq >> 2) & 1);
      const uint32_t base = vtb + dim0 * tRowB + 2 * kpos;
      lds_st<u32x2_t>(base + 0 * tRowB, u32x2_t{__builtin_amdgcn_perm(R1.x, R0.x, 0x05040100u),
                                                 __builtin_amdgcn_perm(R3.x, R2.x, 0x05040100u)});
      lds_st<u32x2_t>(base + 1 * tRowB, u32x2_t{__builtin_amdgcn_perm(R1.x, R0.x, 0x07060302u),
                                                 __builtin_amdgcn_perm(R3.x, R2.x, 0x07060302u)});
      lds_st<u32x2_t>(base + 2 * tRowB, u32x2_t{__builtin_amdgcn_perm(R1.y, R0.y, 0x05040100u),
                                                 __builtin_amdgcn_perm(R3.y, R2.y, 0x05040100u)});
      lds_st<u32x2_t>(base + 3 * tRowB, u32x2_t{__builtin_amdgcn_perm(R1.y, R0.y, 0x07060302u),
                                                 __builtin_amdgcn_perm(R3.y, R2.y, 0x07060302u)});
    }

    // ---- S^T = K~ Q~^T: key rows gathered by code -------------------------
    // lane (n16, kg) supplies key 16 mt + n16, dims 32 c + 8 kg.. = sub 4 c + kg
    float4_t sacc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint32_t kw[4] = {kc[mt].x, kc[mt].y, kc[mt].z, kc[mt].w};
      half8_t kv[4], kl[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t code = __builtin_amdgcn_ubfe(kw[c], 8u * kg, 8u);
        kv[c] = lds_ld<half8_t>((code << 8) | kbase);
        kl[c] = lds_ld<half8_t>((code << 7) + kbase_lo);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
        // small terms first: lo . hi, hi . lo, then hi . hi
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kl[c], qb[nt][c], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv[c], ql[nt][c], acc, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv[c], qb[nt][c], acc, 0, 0, 0);
        sacc[mt][nt] = acc;
      }
      __builtin_amdgcn_sched_barrier(0);  // one key group's gathered rows live at a time
    }
    if (tb + tKT < s_hi) load_codes(tb + tKT, kc, vc);
    // sacc[mt][nt][i]: query row 16 nt + n16, key tb + 16 mt + 4 kg + i

    // ---- masks and lazy online softmax ------------------------------------
    if (!(tb >= full_lo && tb + tKT <= full_hi)) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = tb + 16 * mt + 4 * kg + i;
            if (!(t >= rlo[nt] && t < rhi[nt])) sacc[mt][nt][i] = -INFINITY;
          }
    }
    float tmx[2];
    bool over = false;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[mt][nt][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      tmx[nt] = mx;
      over |= mx > th[nt];
    }
    if (__builtin_amdgcn_ballot_w64(over)) {
      float al[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float mn = fmaxf(m_run[nt], tmx[nt]);
        al[nt] = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[nt] - mn);
        m_run[nt] = mn;
        th[nt] = mn + tLazyMargin;
        mref[nt] = mn == -INFINITY ? 0.f : mn;
        lsum[nt] *= al[nt];
      }
      // rescale O: its rows are laid out as (4 kg + i) per M tile
      wave_sync_lds();
      if (kg == 0) {
        lds_st<float>(tAl + (wave * 32 + n16) * 4, al[0]);
        lds_st<float>(tAl + (wave * 32 + 16 + n16) * 4, al[1]);
      }
      wave_sync_lds();
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const float4_t a4 = lds_ld<float4_t>(tAl + (wave * 32 + 16 * mt + 4 * kg) * 4);
#pragma unroll
        for (int nd = 0; nd < 8; ++nd) oacc[mt][nd] *= a4;
      }
    }
    // p (fp16): ph[nt][mt][i] = row 16 nt + n16, key 16 mt + 4 kg + i
    half4_t ph[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ph[nt][mt][i] = (_Float16)__builtin_amdgcn_exp2f(sacc[mt][nt][i] - mref[nt]);
          lsum[nt] += (float)ph[nt][mt][i];  // the denominator of exactly the weights used
        }
      }
    }
    __syncthreads();  // the V^T tile is complete

    // ---- O += P V ---------------------------------------------------------
    // A: p of rows 16 mt + n16; the lane's K slots 8 kg + 4 h + i of key
    // chunk kc2 hold keys 32 kc2 + 16 h + 4 kg + i, which are its own score
    // registers; B: V^T rows (dims) 16 nd + n16 at the same key positions
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2) {
      half8_t pa[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const half4_t a0 = ph[mt][2 * kc2], a1 = ph[mt][2 * kc2 + 1];
        pa[mt] = half8_t{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      }
#pragma unroll
      for (int nd = 0; nd < 8; ++nd) {
        const half8_t vb = lds_ld<half8_t>(vtb + (16 * nd + n16) * tRowB + 2 * (32 * kc2 + 8 * kg));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          oacc[mt][nd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[mt], vb, oacc[mt][nd], 0, 0, 0);
      }
    }
  };

  __syncthreads();  // the codebook tables are complete
  if (s_lo < s_hi) {
    load_codes(s_lo, kc, vc);
    uint32_t vtb = tVT;
    for (int tb = s_lo; tb < s_hi; tb += tKT) {
      tile(tb, vtb);
      vtb ^= tVT ^ (tVT + tD * tRowB);
    }
  }

  // ---- partials: (m, l, acc[128]) per row ------------------------------------
  // generic split layout: [(b, g)][row tile][split][row][D + 2]
  float* const pbase = part + (((size_t)bg * p.n_rt + rt) * p.n_split + split) * tRT * (tD + 2);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float l = lsum[nt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int r = 32 * wave + 16 * nt + n16;
    if (kg == 0 && rvalid[nt]) {
      pbase[(size_t)r * (tD + 2)] = m_run[nt];
      pbase[(size_t)r * (tD + 2) + 1] = l;
    }
  }
  // O rows 32 wave + 16 mt + 4 kg + i, dims 16 nd + n16
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * wave + 16 * mt + 4 * kg + i;
      if (gr0 + r < p.GS) {
        float* const op = pbase + (size_t)r * (tD + 2) + 2;
#pragma unroll
        for (int nd = 0; nd < 8; ++nd) op[16 * nd + n16] = oacc[mt][nd][i];
      }
    }
}

}  // namespace

bool tile_plan(int B, int Hq, int Sq, int D, int Hkv, int S_cap, int window, int dk, int dv, int n_c,
               TileParams* tp) {
  if (D != tD || dk != 8 || dv != 4 || n_c < 1 || n_c > 256) return false;
  if (B <= 0 || Hq <= 0 || Sq <= 0 || Hkv <= 0 || S_cap <= 0 || Hq % Hkv) return false;
  const long long G = Hq / Hkv, GS = G * Sq;
  if (GS < 64) return false;  // few query rows per key: the streaming kernels fit better
  const long long n_rt = (GS + tRT - 1) / tRT;
  const long long units = (long long)B * Hkv * n_rt;
  const long long max_range = window > 0 ? std::min<long long>(S_cap, (long long)Sq + window - 1) : S_cap;
  // about 256 workgroups (one per CU), at least 4 key tiles per split
  long long n_split = (256 + units - 1) / units;
  n_split = std::max<long long>(1, std::min<long long>(n_split, max_range / (4 * tKT)));
  if (units > 0x7fffffffLL || n_split > 65535) return false;
  if (tp) {
    tp->B = B; tp->Hq = Hq; tp->Sq = Sq; tp->Hkv = Hkv; tp->S_cap = S_cap; tp->n_c = n_c;
    tp->G = (int)G; tp->GS = (int)GS; tp->n_rt = (int)n_rt; tp->n_split = (int)n_split;
    tp->window = window;
  }
  return true;
}

size_t tile_workspace_bytes(int B, int Hq, int Sq, int D, int Hkv, int S_cap, int window) {
  TileParams tp;
  if (!tile_plan(B, Hq, Sq, D, Hkv, S_cap, window, 8, 4, 256, &tp)) return 0;
  return (size_t)B * Hkv * tp.n_rt * tp.n_split * tRT * (tD + 2) * sizeof(float);
}

hipError_t launch_attend_tile(const AttendArgs& a, TileParams tp, hipStream_t st) {
  tp.smooth_rows = a.smooth_rows;
  tp.transform = a.transform;
  tp.causal = a.causal;
  tp.fold = (a.transform ? WhtNorm<tD>::value : 1.f) * a.scale_log2e;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(attend_tile_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)tLdsBytes);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)(a.B * a.Hkv * tp.n_rt), (unsigned)tp.n_split);
  hipLaunchKernelGGL(attend_tile_kernel, grid, dim3(tThreads), tLdsBytes, st, a.q, a.k_codes, a.k_codebook,
                     a.smooth, a.v_codes, a.v_codebook, a.kv_lens, a.partials, tp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the generic split merge, with 128-row groups
  AttParams mp{};
  mp.B = a.B; mp.Hq = a.Hq; mp.Sq = a.Sq; mp.Hkv = a.Hkv; mp.S_cap = a.S_cap;
  mp.G = tp.G; mp.rows = tp.GS; mp.R = tRT; mp.n_rgroups = tp.n_rt; mp.n_split = tp.n_split;
  return launch_attend_merge(a, mp, st);
}

}  // namespace vq
