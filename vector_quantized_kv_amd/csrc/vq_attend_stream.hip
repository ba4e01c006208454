// Persistent streaming attention from product-VQ codes (gfx950): head dim
// 128, key sub_dim 8 (16 key codes per token), value sub_dim 4 (32 value
// codes per token).
//
// Method ("Metal Kernels API" page, "Fused SDPA", metal_fused_sdpa;
// "veloxquant_mlx.cache.vecinfer_cache module" page, fused_sdpa): the query
// gets the dual transform q~ = (q * s) . H, the score of key t is the sum
// over sub-vectors j of q~[j] . C_k[code_j(t)] (equal to q . K_hat_t), read
// from a per-unit table of query-centroid products; the softmax runs online
// in base 2 over split chunks, and the output accumulates p_t C_v[codes of t].
//
// Work split.  A unit is (batch row b, kv head g, group of 4 query rows);
// query row rho of a kv head is (position rho / G, head g * G + rho % G).
// A unit's keys are the union of its rows' valid ranges.  Units are laid
// end to end into one token space of T = sum of unit lengths, and each
// persistent workgroup takes one equal chunk of it (at least 512 keys), so
// ragged lengths and masks cost no imbalance.  The unit prefix is computed
// on the device from kv_lens by wave 0 of every workgroup, with wave scans.  The workgroup walks its
// chunk one unit segment at a time: it builds the unit's score table in
// LDS, its 8 waves claim the segment's 64-key blocks from an LDS counter,
// and the waves' partials (m, l, acc) are combined in LDS into slot c + u
// of (chunk c, unit u) (distinct for all overlapping pairs since chunks and
// units are both ordered).  The merge kernel combines the slots of each
// unit.  While the waves stream a segment, wave 0 writes the query rows of
// the chunk's next unit into a second LDS buffer, so the next table build
// does not wait on global memory.
//
// LDS holds the score table LUT[code][j][row] (fp32, 256 B per code, 64 KiB)
// and the value codebook as fp16 rows replicated 32 times ([code][replica][4
// halves], 64 KiB).  For the scores a lane reads its key's 16 sub-vectors in
// an order rotated by lane mod 16, so the 16 lanes served together read 16
// distinct j (distinct bank quads); for the values it reads replica
// (lane mod 32), so the 32 lanes served together hit distinct banks.  The
// LDS byte address of a gathered row has the code in byte 1, so one v_perm
// per code both extracts the code byte and forms the address.
//
// 4-bit codes (at most 16 centroids): the score table is built for the 16
// codes into scratch, then expanded into a byte-pair table LUT2[byte][slot]
// [row] = LUT[byte & 15][2 p][row] + LUT[byte >> 4][2 p + 1][row] (p = slot
// mod 8, slots p and p + 8 duplicated so 16 lanes read 16 distinct bank
// quads): a key's 8 code bytes need 8 gathers and 28 adds.
//
// Per 64-key block and wave (lane = key for the scores):
//   scores  16 b128 table gathers and 60 fp32 adds: 4 rows at once.
//   softmax lazy: the running max m_r moves only when a score exceeds it by
//           more than 8 (log2 units), so p <= 256 is exact enough in fp16
//           and the usual block needs no cross-lane work.
//   values  8 x 2 v_mfma_f32_16x16x32_f16: M = (row, e), N = 16 value
//           sub-vectors (even / odd in two tiles), K = (2 keys, e') where
//           K group g of instruction q takes keys 4 (2q) + g, 4 (2q + 1) + g
//           (so each value-code load of the wave is one 128-byte span), with
//           A[(r,e)][(t,e')] = p_r(t) [e == e'] built by 4 v_perm from the
//           staged p (rounded to nearest; the row sums add the rounded p),
//           and B = two gathered value rows taken as they are.
#include "vq_internal.h"
#include "vq_lane.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace vq {
namespace {

constexpr int kW = 8;                  // waves per workgroup (2 per SIMD)
constexpr int kThreads = kW * 64;
constexpr int kD = 128;
constexpr int kRows = 4;               // query rows per unit
constexpr int kSlot = kRows * kD + 2 * kRows;  // floats per partial slot
constexpr uint32_t kLut = 0;           // [256][16][4] fp32 score table
constexpr uint32_t kValTab = 65536;    // [256][32][4] fp16
constexpr uint32_t kPStage = 131072;   // [wave][row][72] fp16
constexpr uint32_t kPRow = 144;        // bytes per staged row (64 fp16 + pad)
constexpr uint32_t kPWave = kRows * kPRow;
constexpr uint32_t kQs = kPStage + kW * kPWave;  // [2][row][128] fp32 query rows
constexpr uint32_t kCbk = kQs + 2 * kRows * kD * 4;  // [256][8] fp32 key codebook
constexpr uint32_t kScan = kCbk + 256 * 8 * 4;
constexpr int kMaxUnits = 1791;        // units whose prefix fits in LDS (and B <= U)
constexpr uint32_t kLens = kScan + 64;  // int lens[B], clamped to [0, S_cap]
constexpr uint32_t kPrefix = kLens + 4 * (kMaxUnits + 1);  // int prefix[U + 1]
constexpr float kLazyMargin = 8.f;
constexpr int kMaxChunks = 4096;       // partial slots reserved for chunks (>= workgroups)
// Keys charged for a segment switch when chunks are planned: the combine,
// the next table build and the refill of the load pipeline cost about as
// much time as streaming this many keys.
constexpr int kSegCharge = 2048;
// Keys charged, in the decode step, to the chunk holding a unit's last key
// for the encode of the unit's new token (about 3 us of that workgroup's
// setup; 1536 measured best among 1024 .. 3072).
constexpr int kAppendCharge = 1536;
// int slots of the scan area: 0..3 the chunk plan, kW the block-claim
// counter, kQExp and kQExp + 1 the exponents of the two query buffers
constexpr int kQExp = kW + 4;
constexpr int kMaxGrid = 256;          // persistent workgroups (one per CU)
constexpr uint32_t kWaveMax = kPrefix + 4 * (kMaxUnits + 1);  // float [kW]
constexpr uint32_t kLdsBytes = kWaveMax + 4 * kW;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer descriptor (gfx9 family): 32-bit data format, so
// that untyped loads are range checked against num_records.
constexpr int kBufWord3 = 0x00020000;

// Keeps the compiler from reordering memory accesses across this point;
// emits no instruction.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round
// trips): row_shr 1, 2, 4, 8 scan each row of 16 lanes, then row_bcast 15
// and 31 carry the row totals into the rows above.
__device__ __forceinline__ int wave_scan_int(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false); // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false); // row_bcast:31 -> rows 2, 3
  return v;
}

// Sum over the wave, as a wave-uniform value.
__device__ __forceinline__ int wave_total_int(int v) {
  return __builtin_amdgcn_readlane(wave_scan_int(v), 63);
}

// Maximum over the wave with the same DPP pattern, as a wave-uniform value;
// lanes shifted in from outside a row (or in rows not written) keep -inf.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max_step(float v) {
  const float o = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v),
                                                             CTRL, ROWS, 0xf, false));
  return fmaxf(v, o);
}
__device__ __forceinline__ float wave_max_u(float v) {
  v = dpp_max_step<0x111, 0xf>(v);
  v = dpp_max_step<0x112, 0xf>(v);
  v = dpp_max_step<0x114, 0xf>(v);
  v = dpp_max_step<0x118, 0xf>(v);
  v = dpp_max_step<0x142, 0xa>(v);
  v = dpp_max_step<0x143, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over the wave with the same DPP pattern, as a wave-uniform value.
template <int CTRL, int ROWS, bool BOUND>
__device__ __forceinline__ float dpp_add_step(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, BOUND));
}
__device__ __forceinline__ float wave_total_f(float v) {
  v = dpp_add_step<0x111, 0xf, true>(v);
  v = dpp_add_step<0x112, 0xf, true>(v);
  v = dpp_add_step<0x114, 0xf, true>(v);
  v = dpp_add_step<0x118, 0xf, true>(v);
  v = dpp_add_step<0x142, 0xa, false>(v);
  v = dpp_add_step<0x143, 0xc, false>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One cross-lane Walsh-Hadamard butterfly over lane bit M: returns
// sg x + x(lane ^ M) with sg = -1 where lane bit M is set, +1 elsewhere
// (the same fma as with a shuffle), without a trip through LDS:
//   M = 4   DPP row_shl:4 into banks 0, 2 and row_shr:4 into banks 1, 3;
//   M = 8   DPP row_ror:8;
//   M = 16  v_permlane16_swap of x with itself gives (own, partner) in the
//           even rows and (partner, own) in the odd rows;
//   M = 32  v_permlane32_swap, the same over the two halves of the wave.
template <int M>
__device__ __forceinline__ float xor_butterfly(float x, float sg) {
  const int xi = __float_as_int(x);
  if constexpr (M == 4) {
    int t = __builtin_amdgcn_update_dpp(0, xi, 0x104, 0xf, 0x5, false);
    t = __builtin_amdgcn_update_dpp(t, xi, 0x114, 0xf, 0xa, false);
    return fmaf(sg, x, __int_as_float(t));
  } else if constexpr (M == 8) {
    return fmaf(sg, x, __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0x128, 0xf, 0xf, false)));
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)xi, (unsigned)xi, false, false);
    return fmaf(sg, __uint_as_float(r[1]), __uint_as_float(r[0]));
  } else {
    static_assert(M == 32, "lane bit");
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)xi, (unsigned)xi, false, false);
    return fmaf(sg, __uint_as_float(r[1]), __uint_as_float(r[0]));
  }
}

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
  const __half2 h = __floats2half2_rn(a, b);
  return *reinterpret_cast<const uint32_t*>(&h);
}

// x * 2^sc split into fp16 parts: hi = fp16(x 2^sc), lo = fp16(x 2^sc - hi).
__device__ __forceinline__ void split_f16(float4 x, int sc, half4_t& hi, half4_t& lo) {
  const float v[4] = {ldexpf(x.x, sc), ldexpf(x.y, sc), ldexpf(x.z, sc), ldexpf(x.w, sc)};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = (_Float16)v[i];
    lo[i] = (_Float16)(v[i] - (float)hi[i]);
  }
}

// Exponent e with |m| in [2^(e-1), 2^e) for the largest magnitude m (0 for 0).
__device__ __forceinline__ int mag_exp(float m) {
  return m > 0.f ? __builtin_amdgcn_frexp_expf(m) : 0;
}

// LDS accesses by byte address.  The kernel declares no static LDS, so the
// dynamic area it uses starts at LDS address 0.
typedef __attribute__((address_space(3))) uint8_t lds_byte;
template <typename T>
__device__ __forceinline__ T lds_ld(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(
      reinterpret_cast<const lds_byte*>((size_t)addr));
}

// Valid key range [lo, hi) of query row rho (clamped to the rows that exist)
// in a batch row of len keys: the causal and sliding-window masks.
__device__ __forceinline__ void row_range(const StreamParams& p, int len, int rho, int& lo,
                                          int& hi) {
  rho = rho < p.GS ? rho : p.GS - 1;
  const int qa = len - p.Sq + (int)fast_div((uint32_t)rho, p.div_g);
  int h = p.causal ? (qa + 1 < len ? qa + 1 : len) : len;
  int l = p.window > 0 ? qa - p.window + 1 : 0;
  h = h > 0 ? h : 0;
  l = l > 0 ? l : 0;
  lo = l;
  hi = h > l ? h : l;
}

// unit u -> (b * H_kv + g, row group, batch row b)
__device__ __forceinline__ void unit_coords(const StreamParams& p, int u, int& bg, int& rg, int& b) {
  bg = (int)fast_div((uint32_t)u, p.div_nrg);
  rg = u - bg * p.n_rg;
  b = (int)fast_div((uint32_t)bg, p.div_hkv);
}

// Keys of unit u: from the first row's lower bound to the last row's upper
// bound (both are nondecreasing in rho).
__device__ __forceinline__ int unit_len(const StreamParams& p, const int* lens, int u) {
  int bg, rg, b;
  unit_coords(p, u, bg, rg, b);
  const int len = lens[b];
  int lo0, hi0, lo3, hi3;
  row_range(p, len, 4 * rg, lo0, hi0);
  row_range(p, len, 4 * rg + 3, lo3, hi3);
  return hi3 > lo0 ? hi3 - lo0 : 0;
}

// BITS: width of the key and value codes, 8 (one per byte) or 4 (two per
// byte, the even sub-vector in the low nibble).
// APPEND: the decode step's append runs in the same launch.  Every row b
// has one new token, k_new / v_new [B, H_kv, 1, D], whose codes go to slot
// len_b - 1 of the caches before the keys are read.  The workgroup holding
// a unit's last key encodes that unit's new token during its setup (waves
// 1..3 the key, 4..7 the value, while wave 0 prepares the query rows), with
// the arithmetic of the encode kernels (smoothing x / s, the same rotation
// butterflies, fp32 squared distances summed in order, the lowest index on
// ties), and stores its codes before any wave loads that key.
template <int BITS, bool APPEND>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_stream_kernel(
    const __half* __restrict__ q, uint8_t* k_codes,
    const float* __restrict__ k_codebook, const float* __restrict__ smooth,
    uint8_t* v_codes, const float* __restrict__ v_codebook,
    const int32_t* __restrict__ kv_lens, int* __restrict__ header, float* __restrict__ part,
    const float* __restrict__ qpre, const __half* __restrict__ k_new, const __half* __restrict__ v_new,
    StreamParams p) {
  extern __shared__ __align__(16) uint8_t lds[];
  constexpr uint32_t kKRow = 16 * BITS / 8, kVRow = 32 * BITS / 8;  // code bytes per token
  constexpr int kVR = BITS == 8 ? 16 : 4;  // value-code registers per block and lane
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int* const scan = reinterpret_cast<int*>(lds + kScan);  // small shared ints (see kScan)

  // Query rows of unit uq: dual transform, scaled, into LDS buffer qbuf
  // (run by wave 0), in two halves so that the loads can be issued early.
  // Lane (bq = lane / 4, row ir = lane % 4) holds dims 4 bq + e and
  // 64 + 4 bq + e (e = 0..3) of row ir.
  struct QueryRaw {
    uint2 q[2];
    float4 s[2];
  };
  auto query_load = [&](int uq) {
    QueryRaw r;
    int bgq, rgq, bq_b;
    unit_coords(p, uq, bgq, rgq, bq_b);
    const int gq = bgq - bq_b * p.Hkv;
    // (with the append, lane values re-derived here rather than hoisted:
    // the registers are short)
    int ql = lane;
    if constexpr (APPEND) asm volatile("" : "+v"(ql));
    const int bq = ql >> 2, ir = ql & 3;
    const int rho = 4 * rgq + ir;
    const int rc = rho < p.GS ? rho : p.GS - 1;
    const int ip = (int)fast_div((uint32_t)rc, p.div_g);
    const int h = gq * p.G + rc - ip * p.G;
    const size_t qrow = ((size_t)(bq_b * p.Hq + h) * p.Sq + ip) * kD;
    if (qpre) {
      // rows already dual-transformed (explicit matrix): fp32, in the s slots
#pragma unroll
      for (int k = 0; k < 2; ++k) r.s[k] = *reinterpret_cast<const float4*>(qpre + qrow + 64 * k + 4 * bq);
      return r;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) r.q[k] = *reinterpret_cast<const uint2*>(q + qrow + 64 * k + 4 * bq);
    if (smooth) {
      const float* sp = smooth + (p.smooth_rows == 1 ? 0 : gq) * kD;
#pragma unroll
      for (int k = 0; k < 2; ++k) r.s[k] = *reinterpret_cast<const float4*>(sp + 64 * k + 4 * bq);
    }
    return r;
  };
  auto query_finish = [&](const QueryRaw& r, int uq, int qbuf) {
    const int rgq = uq - (int)fast_div((uint32_t)uq, p.div_nrg) * p.n_rg;
    const int bq = lane >> 2, ir = lane & 3;
    const int rho = 4 * rgq + ir;
    float x[8];
    if (qpre) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        x[4 * k] = r.s[k].x; x[4 * k + 1] = r.s[k].y; x[4 * k + 2] = r.s[k].z; x[4 * k + 3] = r.s[k].w;
      }
    } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float2 f0 = __half22float2(*reinterpret_cast<const __half2*>(&r.q[k].x));
      const float2 f1 = __half22float2(*reinterpret_cast<const __half2*>(&r.q[k].y));
      x[4 * k] = f0.x; x[4 * k + 1] = f0.y; x[4 * k + 2] = f1.x; x[4 * k + 3] = f1.y;
    }
    }
    if (smooth && !qpre) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        x[4 * k] *= r.s[k].x; x[4 * k + 1] *= r.s[k].y; x[4 * k + 2] *= r.s[k].z; x[4 * k + 3] *= r.s[k].w;
      }
    }
    if (p.transform == 1) {
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
      for (int i = 0; i < 8; ++i) x[i] = xor_butterfly<4>(x[i], (lane & 4) ? -1.f : 1.f);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = xor_butterfly<8>(x[i], (lane & 8) ? -1.f : 1.f);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = xor_butterfly<16>(x[i], (lane & 16) ? -1.f : 1.f);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = xor_butterfly<32>(x[i], (lane & 32) ? -1.f : 1.f);
    }
    const float f = rho < p.GS ? p.fold : 0.f;
    float* const qd = reinterpret_cast<float*>(lds + kQs) + qbuf * kRows * kD;
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] *= f;
      mx = fmaxf(mx, fabsf(x[i]));
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
      *reinterpret_cast<float4*>(qd + ir * kD + 64 * k + 4 * bq) =
          make_float4(x[4 * k], x[4 * k + 1], x[4 * k + 2], x[4 * k + 3]);
    const int eq = mag_exp(wave_max_u(mx));  // all lanes take part in the reduction
    if (lane == 0) scan[kQExp + qbuf] = eq;
  };
  auto make_query = [&](int uq, int qbuf) { query_finish(query_load(uq), uq, qbuf); };

  // ---- kernel entry --------------------------------------------------------
  // Every thread loads its share of the two codebooks.  Wave 0 alone plans
  // the chunk, with no barrier and no LDS atomics on the way: the kv lengths
  // (clamped) go to LDS, the unit prefix is a DPP scan over rounds of 64
  // units, the chunk is the equal share [c C0, (c + 1) C0) of the T keys,
  // and the unit holding its first key is found by a ballot.  That unit's
  // query rows are requested before the first barrier, so they arrive while
  // the first segment is set up.  (A wave's LDS accesses execute in issue
  // order, so its reads of lens and pre see its own writes.)
  float4 kq = make_float4(0.f, 0.f, 0.f, 0.f), vq = kq;
  // value codebook as fp16 rows, replicated 32 times; rotated by code so
  // that the 16 lanes of a write hit distinct bank quads
  // 4-bit codes: a byte-pair table instead, entry [byte] = the fp16 rows of
  // codes byte & 15 and byte >> 4 (the two sub-vectors of one code byte),
  // 16 bytes, replicated 16 times ([byte][replica][8 halves], 64 KiB): the
  // 16 lanes of a b128 gather read replicas lane mod 16, distinct bank quads
  float4 vq_hi = make_float4(0.f, 0.f, 0.f, 0.f);
  auto write_val_table = [&]() {
    const int code = tid >> 1;
    const uint32_t h0 = pack_half2(vq.x, vq.y), h1 = pack_half2(vq.z, vq.w);
    uint4 two = make_uint4(h0, h1, h0, h1);
    if constexpr (BITS == 4) two = make_uint4(h0, h1, pack_half2(vq_hi.x, vq_hi.y), pack_half2(vq_hi.z, vq_hi.w));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4*>(lds + kValTab + code * 256 + (tid & 1) * 128 + 16 * ((i + code) & 7)) = two;
  };
  // The plan's chain of round trips starts with wave 0's kv length loads, so
  // they are issued first; the codebook loads follow at once, and their
  // values are not touched until the plan is done.
  int lv0 = p.S_cap;
  if (wave == 0 && kv_lens && lane < p.B) lv0 = kv_lens[lane];
  // (unconditional loads, rows past n_c re-read row 0 and are zeroed below:
  // no select on the loaded registers before the plan)
  const bool cb_row = (tid >> 1) < p.n_c;
  kq = reinterpret_cast<const float4*>(k_codebook)[cb_row ? tid : 0];
  // value rows: code tid / 2 (8-bit); codes byte & 15 and byte >> 4 of byte
  // tid / 2 (4-bit pair table; n_c <= 16)
  const int vlo = BITS == 4 ? (tid >> 1) & 15 : tid >> 1, vhi = (tid >> 5) & 15;
  const bool vlo_ok = vlo < p.n_c, vhi_ok = vhi < p.n_c;
  vq = reinterpret_cast<const float4*>(v_codebook)[vlo_ok ? vlo : 0];
  if constexpr (BITS == 4) vq_hi = reinterpret_cast<const float4*>(v_codebook)[vhi_ok ? vhi : 0];
  int* const lens_w = reinterpret_cast<int*>(lds + kLens);
  int* const pre = reinterpret_cast<int*>(lds + kPrefix);
  int* const plan = scan;  // T, start, end, first unit (ints 0..3 of the scan area)
  const int c = blockIdx.x;
  const int G = gridDim.x;
  QueryRaw qraw;
  int quf = -1;  // wave 0: the first unit, whose query rows it requests
  if (wave == 0) {
    for (int b = lane; b < p.B; b += 64) {
      const int lv = b == lane ? lv0 : (kv_lens ? kv_lens[b] : p.S_cap);
      lens_w[b] = lv < 0 ? 0 : (lv > p.S_cap ? p.S_cap : lv);
    }
    lds_order();
    int carry = 0;
    for (int base = 0; base < p.U; base += 64) {
      const int uu = base + lane;
      const int n = uu < p.U ? unit_len(p, lens_w, uu) : 0;
      const int incl = wave_scan_int(n);
      if (uu < p.U) pre[uu] = carry + incl - n;
      if (c == 0 && uu < p.U && n == 0) {
        header[2 * uu] = 0;       // an empty unit has no partials
        header[2 * uu + 1] = -1;
      }
      carry += __builtin_amdgcn_readlane(incl, 63);
    }
    const int Tw = carry;         // T <= U * S_cap < 2^30 is checked on the host
    if (lane == 0) pre[p.U] = Tw;
    lds_order();
    // Chunks are equal shares of a virtual key space in which every unit
    // after the first is preceded by p.charge virtual keys (the cost of a
    // segment switch: combine, table build, refill of the load pipeline, in
    // keys): unit u owns virtual [vs(u) - charge [u > 0], vs(u) + len) with
    // vs(u) = pre[u] + charge u, and virtual y in it maps to key
    // pre[u] + max(0, y - vs(u)).  These spans tile the virtual space (an
    // empty unit's span maps to the next unit's first key), so every key
    // falls in exactly one chunk.  With the decode step's append, every span
    // also ends in p.charge_end virtual keys (the encode of the unit's new
    // token, done by the workgroup holding its last key): then vs(u) =
    // pre[u] + (charge + charge_end) u, the span is [vs(u) - charge [u > 0],
    // vs(u) + len + charge_end), and y maps to key pre[u] +
    // min(len, max(0, y - vs(u))).
    const int V = Tw + p.charge * (p.U - 1) + p.charge_end * p.U;
    const int C0 = max(p.cmin, (V + G - 1) / G);
    const int ys = c * C0 < V ? c * C0 : V;
    const int ye = min(V, ys + C0);
    int st = Tw, en = Tw, uf = 0;
    if (ys < V) {
      bool found_s = false;
      for (int base = 0; base < p.U; base += 64) {
        const int uu = base + lane;
        bool hs = false, he = false;
        int a0 = 0, vs = 0, ln = 0;
        if (uu < p.U) {
          a0 = pre[uu];
          ln = pre[uu + 1] - a0;
          vs = a0 + (p.charge + p.charge_end) * uu;
          const int lo = uu > 0 ? vs - p.charge : vs, hi = vs + ln + p.charge_end;
          hs = lo <= ys && ys < hi;
          he = lo < ye && ye <= hi;   // the unit holding the chunk's last key
        }
        const uint64_t ms = __builtin_amdgcn_ballot_w64(hs);
        const uint64_t me = __builtin_amdgcn_ballot_w64(he);
        if (ms && !found_s) {
          const int l = (int)__builtin_ctzll(ms);
          uf = base + l;
          st = __builtin_amdgcn_readlane(a0 + min(ln, max(0, ys - vs)), l);
          found_s = true;
        }
        if (me) {
          const int l = (int)__builtin_ctzll(me);
          en = __builtin_amdgcn_readlane(a0 + min(ln, max(0, ye - vs)), l);
          break;
        }
      }
      if (st >= en) {
        st = en = Tw;  // the chunk holds switch cost only
      } else {
        // the first unit with a key at or past st: skips empty units, and a
        // unit of which the chunk holds only the append charge
        while (pre[uf + 1] <= st) ++uf;
        quf = uf;
      }
    }
    if (lane == 0) {
      plan[0] = Tw;
      plan[1] = st;
      plan[2] = en;
      plan[3] = uf;
    }
  }
  // opaque to the compiler: the codebook conversions stay below the plan
  asm volatile("" : "+v"(kq.x), "+v"(kq.y), "+v"(kq.z), "+v"(kq.w));
  asm volatile("" : "+v"(vq.x), "+v"(vq.y), "+v"(vq.z), "+v"(vq.w));
  if constexpr (BITS == 4) asm volatile("" : "+v"(vq_hi.x), "+v"(vq_hi.y), "+v"(vq_hi.z), "+v"(vq_hi.w));
  if (!cb_row) kq = make_float4(0.f, 0.f, 0.f, 0.f);
  if (!vlo_ok) vq = make_float4(0.f, 0.f, 0.f, 0.f);
  if (!vhi_ok) vq_hi = make_float4(0.f, 0.f, 0.f, 0.f);
  {
    *reinterpret_cast<float4*>(lds + kCbk + 16 * tid) = kq;
    // per-wave maximum magnitude of the key codebook
    const float kmx = wave_max_u(fmaxf(fmaxf(fabsf(kq.x), fabsf(kq.y)), fmaxf(fabsf(kq.z), fabsf(kq.w))));
    if (lane == 0) reinterpret_cast<float*>(lds + kWaveMax)[wave] = kmx;
    write_val_table();
  }
  // the first unit's query rows are requested after the codebook stores, so
  // that those stores wait for the codebook loads only; they arrive while
  // every wave sets up its first segment
  if (wave == 0 && quf >= 0) qraw = query_load(quf);
  __syncthreads();
  const int* const lens = lens_w;
  // magnitude exponent of the key codebook
  int ecb;
  {
    const float* wm = reinterpret_cast<const float*>(lds + kWaveMax);
    float mx = 0.f;
#pragma unroll
    for (int w = 0; w < kW; ++w) mx = fmaxf(mx, wm[w]);
    ecb = mag_exp(mx);
  }
  const int T = __builtin_amdgcn_readfirstlane(plan[0]);
  const int start = __builtin_amdgcn_readfirstlane(plan[1]);
  const int end = __builtin_amdgcn_readfirstlane(plan[2]);
  int u = __builtin_amdgcn_readfirstlane(plan[3]);
  if (start >= T) return;
  // the first unit's query rows (requested before the barrier) into buffer
  // 0, before anything else is issued, so that their waits cover nothing
  // but those loads; later units' rows are written during the previous
  // segment's streaming
  if (wave == 0) query_finish(qraw, u, 0);

  // ---- lane constants ------------------------------------------------------
  // Score gathers: at step k = 4 a + b the lane reads sub-vector
  // j = 4 ((a + rdw) mod 4) + (b + rb) mod 4 with (rdw, rb) = lane mod 16, so
  // the 16 lanes served together read 16 distinct j: 16 distinct bank
  // quads of the [code][j][row] table, whatever the codes.  jt[a] holds the
  // four byte offsets 16 j of steps (a, b), sel[b] the v_perm selector that
  // places the code byte of sub-vector j above that offset.
  const int rdw = (lane >> 2) & 3, rb = lane & 3;
  const uint32_t rot1 = (rdw & 1) ? ~0u : 0u, rot2 = (rdw & 2) ? ~0u : 0u;
  uint32_t jt[4], sel[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      w |= (uint32_t)(16 * (4 * ((a + rdw) & 3) + ((b + rb) & 3))) << (8 * b);
    jt[a] = w;
  }
  if constexpr (BITS == 4) {
    // pair table [byte][slot][row]: at step k = 4 a + b the lane reads byte
    // pair p = 4 ((a + rdw) mod 2) + (b + rb) mod 4 (sub-vectors 2p, 2p + 1)
    // from slot p + 8 ((lane / 8) mod 2), 16 distinct slots over 16 lanes
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        w |= (uint32_t)(16 * (4 * ((a + rdw) & 1) + ((b + rb) & 3) + 8 * ((lane >> 3) & 1))) << (8 * b);
      jt[a] = w;
    }
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) sel[b] = 0x0c0c0000u | ((4u + ((b + rb) & 3)) << 8) | (uint32_t)b;
  // 4 x 4 byte transpose across a lane quad (4-bit value codes): selectors
  // of its two v_perm steps at quad position lane mod 4
  const uint32_t tsel1 = (lane & 3) < 2 ? 0x05040100u : 0x03020706u;
  const uint32_t tsel2 = (lane & 1) ? 0x03070105u : 0x06020400u;
  // value replica + 64 KiB: 8-byte rows, replica lane mod 32 (8-bit); 16-byte
  // pair rows, replica lane mod 16 (4-bit)
  const uint32_t vbase = BITS == 8 ? (uint32_t)(lane & 31) * 8u | (1u << 16) : (uint32_t)(lane & 15) * 16u | (1u << 16);
  const int e_a = lane & 3;          // A operand of the value MFMA: row (rA, e_a)
  const int rA = (lane & 15) >> 2;
  const int grp16 = lane >> 4;       // K group of the 16x16x32 operands
  const uint32_t sa0 = e_a == 0 ? 0x0c0c0100u : (e_a == 1 ? 0x01000c0cu : 0x0c0c0c0cu);
  const uint32_t sa1 = e_a == 2 ? 0x0c0c0100u : (e_a == 3 ? 0x01000c0cu : 0x0c0c0c0cu);
  const uint32_t sa2 = e_a == 0 ? 0x0c0c0302u : (e_a == 1 ? 0x03020c0cu : 0x0c0c0c0cu);
  const uint32_t sa3 = e_a == 2 ? 0x0c0c0302u : (e_a == 3 ? 0x03020c0cu : 0x0c0c0c0cu);
  uint8_t* const ps = lds + kPStage + wave * kPWave;
  float* const red = reinterpret_cast<float*>(lds + kLut);  // [kW][kSlot], over the table
  int* const claim_ctr = scan + kW;

  int pos = start;
  int qbuf = 0;          // query buffer of the current unit
  while (true) {
    // ---- segment: unit u, chunk positions [pos, seg_end) ----------------
    const int Pu = pre[u], Pn = pre[u + 1];
    const int seg_end = min(end, Pn);
    // the merge finds unit u's partials in slots c_first + u .. c_last + u
    if (tid == 0) {
      if (pos == Pu) header[2 * u] = c;
      if (seg_end == Pn) header[2 * u + 1] = c;
    }
    int bg, rg, bb;
    unit_coords(p, u, bg, rg, bb);
    const int len = lens[bb];
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
    // next nonempty unit of the chunk, if any
    int u_next = -1;
    if (seg_end < end) {
      u_next = u + 1;
      while (pre[u_next + 1] == pre[u_next]) ++u_next;  // pos < T, so one follows
    }

    // code rows of (b, g) behind bounds-checked buffer descriptors: loads of
    // keys at or past S_cap return zeros (those keys are always masked)
    const size_t row_tok = (size_t)bg * p.S_cap;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(k_codes + row_tok * kKRow), (short)0, p.S_cap * kKRow, kBufWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(v_codes + row_tok * kVRow), (short)0, p.S_cap * kVRow, kBufWord3);

    // codes of one block: the lane's key (16 bytes; 8 with 4-bit codes) and,
    // for the value MFMA, the codes of sub-vectors (2n, 2n+1) of keys
    // 4 j + g, j = 0..15 (two bytes; one with 4-bit codes), kept as loaded
    // (one per register) so that the prefetch of the next block is not
    // waited for until that block is processed.  Load j of the wave reads
    // keys 4 j .. 4 j + 3: one contiguous span.
    auto load_codes = [&](int tb, uint4& kc, uint32_t (&vr)[kVR]) {
      if constexpr (BITS == 8) {
        const u32x4_t k4 = __builtin_amdgcn_raw_buffer_load_b128(krs, (uint32_t)(tb + lane) * 16u, 0, 0);
        kc = make_uint4(k4[0], k4[1], k4[2], k4[3]);
        const uint32_t vo = (uint32_t)(tb + grp16) * 32u + 2u * (uint32_t)(lane & 15);
#pragma unroll
        for (int k = 0; k < 16; ++k) vr[k] = __builtin_amdgcn_raw_buffer_load_b16(vrs, vo + 128u * k, 0, 0);
      } else {
        const u32x2_t k2 = __builtin_amdgcn_raw_buffer_load_b64(krs, (uint32_t)(tb + lane) * 8u, 0, 0);
        kc = make_uint4(k2[0], k2[1], 0u, 0u);
        // lane (quad position j, quad m) of a row reads the 4 code bytes
        // 4 m .. 4 m + 3 of keys 4 (4 i + j) + g, i = 0..3; a 4 x 4 byte
        // transpose across the quad (in the stage) then gives each lane its
        // byte 4 m + j of keys 4 (4 i + 0..3) + g
        const uint32_t vo = (uint32_t)(tb + grp16 + 4 * (lane & 3)) * 16u + 4u * (uint32_t)((lane & 15) >> 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[i] = __builtin_amdgcn_raw_buffer_load_b32(vrs, vo + 256u * i, 0, 0);
      }
    };

    // Blocks of the segment are t0 + 64 n.  Wave w takes blocks w and
    // w + kW, then claims the next free block from an LDS counter each time
    // it issues a load, so waves that run ahead take more blocks.  Block i
    // of a wave lives in code buffer i mod 3 and is loaded two blocks ahead,
    // so two blocks are in flight while one is processed; the first two
    // load while the table is built.  Loads for claims past the segment
    // re-read block 0 (cache hits), so every step issues the same loads.
    // a claim is issued one step before its block index is needed, so the
    // atomic's latency hides behind a block
    auto claim_issue = [&]() {
      int v = 0;
      if (lane == 0) v = atomicAdd(claim_ctr, 1);
      return v;
    };
    int pend = 0;
    auto claim = [&]() {
      const int n = __builtin_amdgcn_readfirstlane(pend);
      pend = claim_issue();
      return n;
    };
    auto blk = [&](int n) {
      const int tb = t0 + 64 * n;
      return tb < t1 ? tb : t0;
    };
    // ---- append: this segment holds key len - 1, the unit's new token ----
    // Partial searches: keys on waves 1..3 (lane (r, j): sub-vector j,
    // centroids c = 4 (w - 1) + r + 12 k), values on waves 4..7 (lane
    // (r, j): centroids c = 2 (w - 4) + r + 8 k), each merged over its
    // wave's replicas and written as (distance, index) pairs to the idle
    // query buffer; wave 1 merges them after the next barrier.  The value
    // waves stage the fp32 value codebook in the idle p staging area (each
    // writes the same rows and reads them back in its own issue order).
    const int tn = len - 1;
    const bool has_new = APPEND && tn >= t0 && tn < t1;
    // the first loads cover blocks 0 .. 2 kW - 1: if the new key is among
    // them, they wait until its codes are stored; so do those of wave 1,
    // which stores them (its wait for the stores then covers nothing else)
    const bool defer_loads = has_new && (tn < t0 + 2 * kW * 64 || wave == 1);
    float* const apx = reinterpret_cast<float*>(lds + kQs) + (qbuf ^ 1) * kRows * kD;
    auto merge_pair = [](float& best, int& idx, float ob, int oi) {
      const bool lt = ob < best || (ob == best && oi < idx);
      best = lt ? ob : best;
      idx = lt ? oi : idx;
    };
    // (global accesses through buffer descriptors: a wave-uniform base and a
    // 32-bit lane offset, no per-lane 64-bit addresses held across the loop)
    // The lane index is re-read through an empty asm so that the lane values
    // derived from it are computed here, not hoisted out of the segment loop
    // into registers the streaming loop needs.
    if constexpr (APPEND) {
      if (has_new && wave >= 1) {
        int al = lane;
        asm volatile("" : "+v"(al));
        const int g = bg - bb * p.Hkv;
        float best = INFINITY;
        int idx = 0x7fffffff;
        if (wave <= 3) {
          const int r = al >> 4, jk = al & 15, pt = 4 * (wave - 1) + r;
          const __amdgpu_buffer_rsrc_t kn_rs = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<__half*>(k_new + (size_t)bg * kD), (short)0, kD * 2, kBufWord3);
          const u32x4_t kr = __builtin_amdgcn_raw_buffer_load_b128(kn_rs, (uint32_t)jk * 16u, 0, 0);
          RawHalves<8> raw;
#pragma unroll
          for (int i = 0; i < 4; ++i) raw.w[i] = kr[i];
          float sv[8], x[8];
          if (smooth) {
            const __amdgpu_buffer_rsrc_t sm_rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(smooth + (p.smooth_rows == 1 ? 0 : g) * kD), (short)0, kD * 4, kBufWord3);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const u32x4_t sr = __builtin_amdgcn_raw_buffer_load_b128(sm_rs, (uint32_t)jk * 32u + 16u * h2, 0, 0);
#pragma unroll
              for (int i = 0; i < 4; ++i) sv[4 * h2 + i] = __uint_as_float(sr[i]);
            }
          }
          cvt_raw_f16<8>(raw, x);
          if (smooth) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = x[e] / sv[e];
          }
          if (p.transform == 1) wht<kD, 8>(x, jk);
          const float* cbk = reinterpret_cast<const float*>(lds + kCbk);
          if (pt < p.n_c) idx = pt;
          // unrolled so that several centroid rows are read from LDS at once
#pragma unroll 4
          for (int cc = pt; cc < p.n_c; cc += 12) {
            const float* cr = cbk + cc * 8;
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float df = x[e] - cr[e];
              acc = fmaf(df, df, acc);
            }
            if (acc < best) { best = acc; idx = cc; }
          }
          merge_pair(best, idx, __shfl_xor(best, 32), __shfl_xor(idx, 32));
          merge_pair(best, idx, __shfl_xor(best, 16), __shfl_xor(idx, 16));
          if (al < 16) {
            apx[2 * (16 * (wave - 1) + jk)] = best;
            reinterpret_cast<int*>(apx)[2 * (16 * (wave - 1) + jk) + 1] = idx;
          }
        } else {
          const int r = al >> 5, jv = al & 31, pt = 2 * (wave - 4) + r;
          const __amdgpu_buffer_rsrc_t vn_rs = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<__half*>(v_new + (size_t)bg * kD), (short)0, kD * 2, kBufWord3);
          const u32x2_t vr2 = __builtin_amdgcn_raw_buffer_load_b64(vn_rs, (uint32_t)jv * 8u, 0, 0);
          RawHalves<4> raw;
          raw.w[0] = vr2[0];
          raw.w[1] = vr2[1];
          // rows past n_c read as zeros (outside the descriptor's range)
          const __amdgpu_buffer_rsrc_t cv_rs = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<float*>(v_codebook), (short)0, p.n_c * 16, kBufWord3);
          u32x4_t vrow[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vrow[i] = __builtin_amdgcn_raw_buffer_load_b128(cv_rs, (uint32_t)(al + 64 * i) * 16u, 0, 0);
          float* const vcb = reinterpret_cast<float*>(lds + kPStage);
#pragma unroll
          for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(vcb + 4 * (al + 64 * i)) = vrow[i];
          lds_order();
          float x[4];
          cvt_raw_f16<4>(raw, x);
          if (pt < p.n_c) idx = pt;
#pragma unroll 8
          for (int cc = pt; cc < p.n_c; cc += 8) {
            const float* cr = vcb + cc * 4;
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float df = x[e] - cr[e];
              acc = fmaf(df, df, acc);
            }
            if (acc < best) { best = acc; idx = cc; }
          }
          merge_pair(best, idx, __shfl_xor(best, 32), __shfl_xor(idx, 32));
          if (al < 32) {
            apx[2 * (48 + 32 * (wave - 4) + jv)] = best;
            reinterpret_cast<int*>(apx)[2 * (48 + 32 * (wave - 4) + jv) + 1] = idx;
          }
        }
      }
    }
    // wave 1, after the next barrier: the merged codes of the new token, and
    // their stores (which complete before the table barrier)
    auto append_store = [&]() {
      int al = lane;
      asm volatile("" : "+v"(al));
      const int* const apxi = reinterpret_cast<const int*>(apx);
      float best = INFINITY;
      int idx = 0x7fffffff;
      const int jk = al, jv = al - 32;
      if (al < 16) {
#pragma unroll
        for (int k = 0; k < 3; ++k) merge_pair(best, idx, apx[2 * (16 * k + jk)], apxi[2 * (16 * k + jk) + 1]);
      } else if (al >= 32) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          merge_pair(best, idx, apx[2 * (48 + 32 * k + jv)], apxi[2 * (48 + 32 * k + jv) + 1]);
      }
      // 4-bit codes: the even sub-vector's lane packs its odd neighbour's
      // code (lane + 1, the same row of 16 lanes) into the high nibble
      const int idx_next = __builtin_amdgcn_mov_dpp(idx, 0x101, 0xf, 0xf, false);
      const uint8_t code = BITS == 8 ? (uint8_t)idx : (uint8_t)((idx & 15) | ((idx_next & 15) << 4));
      // slot tn of the (b, g) code rows, through the rows' load descriptors
      if (al < 16) {
        if (BITS == 8 || !(jk & 1))
          __builtin_amdgcn_raw_buffer_store_b8(code, krs, (uint32_t)tn * kKRow + (uint32_t)(BITS == 8 ? jk : jk / 2), 0, 0);
      } else if (al >= 32) {
        if (BITS == 8 || !(jv & 1))
          __builtin_amdgcn_raw_buffer_store_b8(code, vrs, (uint32_t)tn * kVRow + (uint32_t)(BITS == 8 ? jv : jv / 2), 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0);  // the stores are complete before the barrier
    };

    int nA = wave, nB = wave + kW, nC = 0;
    uint4 kcA, kcB, kcC;
    uint32_t vrA[kVR], vrB[kVR], vrC[kVR];
    if (!defer_loads && t0 + 64 * nA < t1) {
      load_codes(blk(nA), kcA, vrA);
      load_codes(blk(nB), kcB, vrB);
    }

    if (tid == 0) *claim_ctr = 2 * kW;
    __syncthreads();  // query rows ready; the previous combine has read the table area
    {
      const float* const qcur = reinterpret_cast<const float*>(lds + kQs) + qbuf * kRows * kD;
      // ---- score table: LUT[code][j][r] = q~_r[8 j .. 8 j + 7] . C_k[code] --
      // on the matrix cores: v_mfma_f32_32x32x8_f16 with M = 32 codes (wave
      // w: codes 32 w ..), N = 32 (j, r) pairs (two tiles: j < 8, j >= 8),
      // K = the 8 dims of a sub-vector.  Both operands are scaled by powers
      // of two into [2^13, 2^14) and split into fp16 high and low parts; the
      // products hi.hi + lo.hi + hi.lo carry the result to fp32 accuracy.
      // 4-bit codes: wave 0 builds the 16-code table into the p staging
      // area; the byte-pair table LUT2[byte][slot][r] = LUT[b & 15][2 p][r] +
      // LUT[b >> 4][2 p + 1][r] (p = slot mod 8) then fills the table area.
      if (BITS == 8 || wave == 0) {
        const int l32 = lane & 31, kh = lane >> 5;
        const int eq = scan[kQExp + qbuf];
        const float* cbk = reinterpret_cast<const float*>(lds + kCbk);
        const float4 a = *reinterpret_cast<const float4*>(cbk + 8 * (32 * wave + l32) + 4 * kh);
        half4_t ahi, alo;
        split_f16(a, 14 - ecb, ahi, alo);
        const int unscale = ecb + eq - 28;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          // column n = l32: sub-vector j = 8 t2 + n / 4, row r = n % 4
          const float4 b = *reinterpret_cast<const float4*>(qcur + (l32 & 3) * kD + 8 * (8 * t2 + (l32 >> 2)) + 4 * kh);
          half4_t bhi, blo;
          split_f16(b, 14 - eq, bhi, blo);
          float16_t d = {};
          d = __builtin_amdgcn_mfma_f32_32x32x8f16(ahi, bhi, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_32x32x8f16(alo, bhi, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_32x32x8f16(ahi, blo, d, 0, 0, 0);
          // element v: code 32 w + 8 (v / 4) + 4 kh + v % 4, column l32
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int code = 32 * wave + 8 * (v >> 2) + 4 * kh + (v & 3);
            if constexpr (BITS == 8)
              *reinterpret_cast<float*>(lds + kLut + code * 256 + 128 * t2 + 4 * l32) = ldexpf(d[v], unscale);
            else if (code < 16)
              *reinterpret_cast<float*>(lds + kPStage + code * 256 + 128 * t2 + 4 * l32) = ldexpf(d[v], unscale);
          }
        }
      }
      if constexpr (BITS == 4) {
        __syncthreads();
        const float* small = reinterpret_cast<const float*>(lds + kPStage);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = tid + kThreads * i;  // (byte, slot) = (e / 16, e mod 16)
          const int byte = e >> 4, pr = e & 7;
          const float4 x = *reinterpret_cast<const float4*>(small + 64 * (byte & 15) + 4 * (2 * pr));
          const float4 y = *reinterpret_cast<const float4*>(small + 64 * (byte >> 4) + 4 * (2 * pr + 1));
          *reinterpret_cast<float4*>(lds + kLut + 16 * e) = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
        }
      }
      if (has_new && wave == 1) append_store();
    }
    __syncthreads();
    // the first loads of a segment whose new key is among them
    if (defer_loads && t0 + 64 * nA < t1) {
      load_codes(blk(nA), kcA, vrA);
      load_codes(blk(nB), kcB, vrB);
    }
    // the next unit's query rows, written while the other waves stream
    if (u_next >= 0 && wave == 0) make_query(u_next, qbuf ^ 1);

    float m[kRows], lsum[kRows], th[kRows], mref[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      m[r] = -INFINITY; th[r] = -INFINITY; mref[r] = 0.f; lsum[r] = 0.f;
    }
    float4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;

    // Software pipeline over the wave's 64-key blocks.  A block's score
    // gathers run while the previous block's value rows (gathered at the
    // end of its own stage) go through the value MFMAs; the code buffers of
    // consecutive blocks alternate between two register sets, so the
    // prefetch of the next block is only waited for when it is used.
    u32x2_t vg[8][4];  // value rows of the block whose value MFMAs are pending
    uint32_t wq[4];    // (8-bit) its packed codes of key pairs 4..7, gathered mid-stage
    u32x4_t vp[8][2];  // (4-bit) its pair-table rows: [key 0 | key 1][sub 2n, sub 2n + 1]
    uint32_t pp[8];    // that block's p, staged into the A operand layout

    auto value_mfmas = [&](auto half) {
#pragma unroll
      for (int k = 4 * decltype(half)::value; k < 4 * decltype(half)::value + 4; ++k) {
        const uint32_t x = pp[k];
        const uint4 au = make_uint4(__builtin_amdgcn_perm(0u, x, sa0), __builtin_amdgcn_perm(0u, x, sa1),
                                    __builtin_amdgcn_perm(0u, x, sa2), __builtin_amdgcn_perm(0u, x, sa3));
        const uint4 b0 = BITS == 8 ? make_uint4(vg[k][0].x, vg[k][0].y, vg[k][1].x, vg[k][1].y)
                                   : make_uint4(vp[k][0][0], vp[k][0][1], vp[k][1][0], vp[k][1][1]);
        const uint4 b1 = BITS == 8 ? make_uint4(vg[k][2].x, vg[k][2].y, vg[k][3].x, vg[k][3].y)
                                   : make_uint4(vp[k][0][2], vp[k][0][3], vp[k][1][2], vp[k][1][3]);
        const half8_t A = *reinterpret_cast<const half8_t*>(&au);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, *reinterpret_cast<const half8_t*>(&b0), acc0,
                                                      0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, *reinterpret_cast<const half8_t*>(&b1), acc1,
                                                      0, 0, 0);
      }
    };
    auto gather_hi = [&]() {
#pragma unroll
      for (int k = 4; k < 8; ++k) {
        const uint32_t w = wq[k - 4];
        vg[k][0] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020400u));
        vg[k][1] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020600u));
        vg[k][2] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020500u));
        vg[k][3] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020700u));
      }
    };
    const std::integral_constant<int, 0> lo_half;
    const std::integral_constant<int, 1> hi_half;

    auto stage = [&](int tb, const uint4& kc, const uint32_t (&vr)[kVR], bool pending) {
      // ---- scores: 16 table rows of 4 fp32 (one per query row), in two
      // halves, each overlapping half of the previous block's value MFMAs
      float4_t sc;
      {
        if constexpr (BITS == 8) {
          // dw[a] = kw[(a + rdw) mod 4]: rotate by rdw bit 0, then by bit 1,
          // with bit selects (no divergent branches)
          const uint32_t kw[4] = {kc.x, kc.y, kc.z, kc.w};
          uint32_t r1[4], dw[4];
#pragma unroll
          for (int a = 0; a < 4; ++a) r1[a] = (kw[(a + 1) & 3] & rot1) | (kw[a] & ~rot1);
#pragma unroll
          for (int a = 0; a < 4; ++a) dw[a] = (r1[(a + 2) & 3] & rot2) | (r1[a] & ~rot2);
          float4_t L[8];
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
              L[4 * a + b] = lds_ld<float4_t>(kLut + __builtin_amdgcn_perm(dw[a], jt[a], sel[b]));
          __builtin_amdgcn_sched_barrier(0);
          if (pending) value_mfmas(lo_half);
          if (pending) gather_hi();
          __builtin_amdgcn_sched_barrier(0);
          sc = ((L[0] + L[1]) + (L[2] + L[3])) + ((L[4] + L[5]) + (L[6] + L[7]));
#pragma unroll
          for (int a = 2; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
              L[4 * (a - 2) + b] = lds_ld<float4_t>(kLut + __builtin_amdgcn_perm(dw[a], jt[a], sel[b]));
          __builtin_amdgcn_sched_barrier(0);
          if (pending) value_mfmas(hi_half);
          sc += ((L[0] + L[1]) + (L[2] + L[3])) + ((L[4] + L[5]) + (L[6] + L[7]));
        } else {
          // 4-bit: the 8 code bytes (sub-vector pairs) of the key, words
          // swapped by rdw bit 0; one pair-table gather per byte
          const uint32_t dw[2] = {(kc.y & rot1) | (kc.x & ~rot1), (kc.x & rot1) | (kc.y & ~rot1)};
          float4_t L[8];
#pragma unroll
          for (int b = 0; b < 4; ++b)
            L[b] = lds_ld<float4_t>(kLut + __builtin_amdgcn_perm(dw[0], jt[0], sel[b]));
          __builtin_amdgcn_sched_barrier(0);
          if (pending) value_mfmas(lo_half);
#pragma unroll
          for (int b = 0; b < 4; ++b)
            L[4 + b] = lds_ld<float4_t>(kLut + __builtin_amdgcn_perm(dw[1], jt[1], sel[b]));
          __builtin_amdgcn_sched_barrier(0);
          if (pending) value_mfmas(hi_half);
          sc = ((L[0] + L[1]) + (L[2] + L[3])) + ((L[4] + L[5]) + (L[6] + L[7]));
        }
      }

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
          const float mn = fmaxf(m[r], wave_max_u(s[r]));
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
      // p rounded to nearest fp16; the row sums take the rounded values, so
      // the weights and their normalizer agree
      uint32_t p01, p23;
      {
        float pr[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r) pr[r] = __builtin_amdgcn_exp2f(s[r] - mref[r]);
        p01 = pack_half2(pr[0], pr[1]);
        p23 = pack_half2(pr[2], pr[3]);
        const float2 f01 = __half22float2(*reinterpret_cast<const __half2*>(&p01));
        const float2 f23 = __half22float2(*reinterpret_cast<const __half2*>(&p23));
        lsum[0] += f01.x; lsum[1] += f01.y; lsum[2] += f23.x; lsum[3] += f23.y;
      }

      // ---- p to the value operand layout through LDS -------------------
      // A wave's LDS accesses execute in issue order, so the reads below see
      // these writes, and the previous block's reads of the same area were
      // issued before them; only the compiler must keep the order.
      lds_order();
      {
        // key 4 q + g is staged at position 16 g + q, so that lane group g
        // finds its keys 4 q + g (q = 0..15) contiguous
        uint8_t* const pw = ps + 2 * (16 * (lane & 3) + (lane >> 2));
        *reinterpret_cast<uint16_t*>(pw + 0 * kPRow) = (uint16_t)p01;
        *reinterpret_cast<uint16_t*>(pw + 1 * kPRow) = (uint16_t)(p01 >> 16);
        *reinterpret_cast<uint16_t*>(pw + 2 * kPRow) = (uint16_t)p23;
        *reinterpret_cast<uint16_t*>(pw + 3 * kPRow) = (uint16_t)(p23 >> 16);
      }
      lds_order();
      const uint4 P0 = *reinterpret_cast<const uint4*>(ps + rA * kPRow + 32 * grp16);
      const uint4 P1 = *reinterpret_cast<const uint4*>(ps + rA * kPRow + 32 * grp16 + 16);
      pp[0] = P0.x; pp[1] = P0.y; pp[2] = P0.z; pp[3] = P0.w;
      pp[4] = P1.x; pp[5] = P1.y; pp[6] = P1.z; pp[7] = P1.w;

      // ---- this block's value rows, consumed by the next stage ---------
      // rows of key pair k: [key 0 sub 2n, key 1 sub 2n, key 0 sub 2n+1, key 1 sub 2n+1]
      uint32_t t4[4];  // (4-bit) byte 4 m + j of keys 4 (4 i + 0..3) + g, per i
      if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t X = vr[i];
          const uint32_t Z = __builtin_amdgcn_perm(
              (uint32_t)__builtin_amdgcn_mov_dpp((int)X, 0x4e, 0xf, 0xf, true), X, tsel1);
          t4[i] = __builtin_amdgcn_perm(
              (uint32_t)__builtin_amdgcn_mov_dpp((int)Z, 0xb1, 0xf, 0xf, true), Z, tsel2);
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if constexpr (BITS == 8) {
          // [code(key 0, 2n), code(key 0, 2n+1), code(key 1, 2n), code(key 1, 2n+1)]
          const uint32_t w = __builtin_amdgcn_perm(vr[2 * k + 1], vr[2 * k], 0x05040100u);
          if (k >= 4) {
            wq[k - 4] = w;
            continue;
          }
          vg[k][0] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020400u));
          vg[k][1] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020600u));
          vg[k][2] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020500u));
          vg[k][3] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020700u));
        } else {
          // one pair-table row per key: its code byte of sub-vectors 2n, 2n + 1
          const uint32_t y = t4[k >> 1];
          const uint32_t s0 = (k & 1) ? 0x0c020600u : 0x0c020400u, s1 = (k & 1) ? 0x0c020700u : 0x0c020500u;
          vp[k][0] = lds_ld<u32x4_t>(__builtin_amdgcn_perm(y, vbase, s0));
          vp[k][1] = lds_ld<u32x4_t>(__builtin_amdgcn_perm(y, vbase, s1));
        }
      }
    };

    if (t0 + 64 * nA < t1) {
      pend = claim_issue();
      bool pending = false;
      for (;;) {
        nC = claim();
        load_codes(blk(nC), kcC, vrC);
        stage(t0 + 64 * nA, kcA, vrA, pending);
        pending = true;
        if (t0 + 64 * nB >= t1) break;
        nA = claim();
        load_codes(blk(nA), kcA, vrA);
        stage(t0 + 64 * nB, kcB, vrB, true);
        if (t0 + 64 * nC >= t1) break;
        nB = claim();
        load_codes(blk(nB), kcB, vrB);
        stage(t0 + 64 * nC, kcC, vrC, true);
        if (t0 + 64 * nA >= t1) break;
      }
      value_mfmas(lo_half);
      if constexpr (BITS == 8) gather_hi();
      value_mfmas(hi_half);
    }

    // ---- combine the waves' partials of the segment into slot c + u -------
    float l[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) l[r] = wave_total_f(lsum[r]);
    __syncthreads();  // every wave is done with the table
    {
      float* sp = red + wave * kSlot;
      const int r = lane >> 4, n = lane & 15;
      *reinterpret_cast<float4*>(sp + r * kD + 8 * n) = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
      *reinterpret_cast<float4*>(sp + r * kD + 8 * n + 4) = make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
      if (lane < kRows) {
        sp[kRows * kD + lane] = lane == 0 ? m[0] : (lane == 1 ? m[1] : (lane == 2 ? m[2] : m[3]));
        sp[kRows * kD + kRows + lane] = lane == 0 ? l[0] : (lane == 1 ? l[1] : (lane == 2 ? l[2] : l[3]));
      }
    }
    __syncthreads();
    {
      // thread -> (row r, dim d)
      const int r = tid >> 7, d = tid & (kD - 1);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kW; ++w) M = fmaxf(M, red[w * kSlot + kRows * kD + r]);
      float Ls = 0.f, A = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kW; ++w) {
          const float mw = red[w * kSlot + kRows * kD + r];
          const float sw = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
          Ls += sw * red[w * kSlot + kRows * kD + kRows + r];
          A += sw * red[w * kSlot + r * kD + d];
        }
      }
      float* gp = part + (size_t)(c + u) * kSlot;
      gp[r * kD + d] = A;
      if (d == 0) {
        gp[kRows * kD + r] = M;
        gp[kRows * kD + kRows + r] = Ls;
      }
    }


    if (u_next < 0) break;
    pos = seg_end;
    u = u_next;
    qbuf ^= 1;
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
  const int c_lo = header[2 * u], n_part = header[2 * u + 1] - c_lo + 1;
  float2 acc = make_float2(0.f, 0.f);
  float L = 0.f;
  if (n_part > 0) {
    const float* base = part + (size_t)(c_lo + u) * kSlot;
    // up to 8 partials per round: their (m, l) and the lane's two
    // accumulator values load together, then fold into the running sums
    float M = -INFINITY;
    for (int j0 = 0; j0 < n_part; j0 += 8) {
      float mj[8], lj[8];
      float2 xj[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool ok = j0 + k < n_part;
        const float* sp = base + (size_t)(j0 + k) * kSlot;
        mj[k] = ok ? sp[kRows * kD + r] : -INFINITY;
        lj[k] = ok ? sp[kRows * kD + kRows + r] : 0.f;
        xj[k] = ok ? *reinterpret_cast<const float2*>(sp + r * kD + 2 * lane) : make_float2(0.f, 0.f);
      }
      float Mn = M;
#pragma unroll
      for (int k = 0; k < 8; ++k) Mn = fmaxf(Mn, mj[k]);
      if (Mn == -INFINITY) continue;
      const float al = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      L *= al;
      acc.x *= al;
      acc.y *= al;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float w = mj[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mj[k] - Mn);
        L += w * lj[k];
        acc.x += w * xj[k].x;
        acc.y += w * xj[k].y;
      }
      M = Mn;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<__half2*>(out + (size_t)row * kD + 2 * lane) =
      __floats2half2_rn(acc.x * inv, acc.y * inv);
}

// CUs of the current device, cached per device (any thread may launch:
// relaxed atomics, and racing threads store the same value).
int cached_cu_count() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

bool stream_plan(int B, int Hq, int Sq, int D, int Hkv, int S_cap, int window, int dk, int dv, int n_c,
                 StreamParams* sp, size_t* lds_bytes, size_t* ws_bytes) {
  if (D != kD || dk != 8 || dv != 4 || n_c < 1 || n_c > 256) return false;
  if (B <= 0 || Hq <= 0 || Sq <= 0 || Hkv <= 0 || S_cap <= 0 || Hq % Hkv) return false;
  const long long G = Hq / Hkv, GS = G * Sq, n_rg = (GS + kRows - 1) / kRows;
  const long long U = (long long)B * Hkv * n_rg;
  if (U > kMaxUnits || U * (long long)S_cap >= (1LL << 30) || S_cap >= (1 << 26)) return false;
  // the persistent grid's fixed cost (table fill, unit prefix, merge) only
  // pays off with enough keys: small problems go to the per-unit kernel
  const long long max_range = window > 0 ? std::min<long long>(S_cap, (long long)Sq + window - 1) : S_cap;
  if (U * max_range < (1LL << 18)) return false;
  if (sp) {
    sp->B = B; sp->Hq = Hq; sp->Sq = Sq; sp->Hkv = Hkv; sp->S_cap = S_cap; sp->n_c = n_c;
    sp->G = (int)G; sp->GS = (int)GS; sp->n_rg = (int)n_rg; sp->U = (int)U; sp->cmin = kW * 64;
    // units of a sliding window usually have equal lengths, which equal
    // shares tend to split at unit starts: charging switches there only
    // breaks that alignment
    sp->charge = window > 0 ? 0 : kSegCharge;
    sp->charge_end = 0;
    sp->div_g = make_fastdiv((uint32_t)G);
    sp->div_nrg = make_fastdiv((uint32_t)n_rg);
    sp->div_hkv = make_fastdiv((uint32_t)Hkv);
  }
  if (lds_bytes) *lds_bytes = kLdsBytes;
  if (ws_bytes) *ws_bytes = stream_workspace_bytes(B, Hq, Sq, D, Hkv);
  return true;
}

size_t stream_workspace_bytes(int B, int Hq, int Sq, int D, int Hkv) {
  if (D != kD || B <= 0 || Hq <= 0 || Sq <= 0 || Hkv <= 0 || Hq % Hkv) return 0;
  const long long G = Hq / Hkv, GS = G * Sq, n_rg = (GS + kRows - 1) / kRows;
  const long long U = (long long)B * Hkv * n_rg;
  const size_t header = ((size_t)U * 8 + 255) / 256 * 256;  // (first, last chunk) per unit
  return header + (size_t)(kMaxChunks + U) * kSlot * sizeof(float);
}

hipError_t launch_attend_stream(const AttendArgs& a, StreamParams sp, size_t lds, hipStream_t st) {
  const int cus = cached_cu_count();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int grid = cus < kMaxGrid ? cus : kMaxGrid;
  sp.smooth_rows = a.smooth_rows;
  sp.transform = a.transform;
  sp.causal = a.causal;
  sp.window = a.window;
  sp.fold = (a.transform == 1 ? WhtNorm<kD>::value : 1.f) * a.scale_log2e;
  sp.charge_end = a.k_new ? kAppendCharge : 0;
  const size_t header_bytes = ((size_t)sp.U * 8 + 255) / 256 * 256;
  int* header = reinterpret_cast<int*>(a.partials);
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.partials) + header_bytes);
  const bool append = a.k_new != nullptr;
  auto kern = a.code_bits == 4 ? (append ? attend_stream_kernel<4, true> : attend_stream_kernel<4, false>)
                               : (append ? attend_stream_kernel<8, true> : attend_stream_kernel<8, false>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, st, a.q, const_cast<uint8_t*>(a.k_codes),
                     a.k_codebook, a.smooth, const_cast<uint8_t*>(a.v_codes), a.v_codebook, a.kv_lens, header,
                     part, a.q_pre, a.k_new, a.v_new, sp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)a.B * a.Hq * a.Sq;
  hipLaunchKernelGGL(stream_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, header,
                     part, a.out, sp);
  return hipGetLastError();
}

}  // namespace vq
