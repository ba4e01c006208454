// Split-K attention read directly from product-VQ key and value codes.
//
// Method ("Metal Kernels API" page, "Fused SDPA", metal_fused_sdpa;
// "veloxquant_mlx.cache.vecinfer_cache module" page, fused_sdpa): the raw
// query gets the dual transform q~ = (q * s) . H, so that
// q~ . K~_t = q . K_hat_t; scores are sums of per-sub-vector query LUT
// entries LUT[j][c] = <q~_j, C_k[c]> gathered by the key codes; softmax runs
// online (base 2, scale and log2(e) folded into the LUT); values are
// gathered from the value codebook by the value codes.
//
// Work decomposition (MI355X): one workgroup per (batch row, kv head,
// row group of up to R query rows, split of the key axis).  The R rows of a
// GQA group share one LUT in LDS laid out [j][code][row], so one code byte
// fetches the score terms of every row with a single LDS read.  Each wave
// owns a stream of 64-key chunks: lane = key for the score, mask and online
// softmax; then lanes re-map to (4-dim slice of the head, key parity) to
// accumulate values.  The four waves and the splits are merged with the
// log-sum-exp rule (flash-decoding); splits are combined by a second kernel.
#include "vq_internal.h"

#include <algorithm>

namespace vq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr size_t kLdsBudget = 160 * 1024;

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

// Reads R consecutive floats (R-aligned in the LDS) with vector loads.
template <int R>
__device__ __forceinline__ void lds_read_row(const float* e, float (&v)[R]) {
  if constexpr (R == 1) {
    v[0] = e[0];
  } else if constexpr (R == 2) {
    const float2 a = *reinterpret_cast<const float2*>(e);
    v[0] = a.x; v[1] = a.y;
  } else {
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      const float4 a = *reinterpret_cast<const float4*>(e + r);
      v[r] = a.x; v[r + 1] = a.y; v[r + 2] = a.z; v[r + 3] = a.w;
    }
  }
}

// LDS carve-up, in floats (the code staging area is counted in bytes / 4).
struct LdsLayout {
  size_t lut, cv, qt, pst, vst, total_floats;
};

__host__ __device__ inline LdsLayout lds_layout(int nsk, int n_c, int dv, int nsv, int R, int D) {
  // every region starts on a 16-byte boundary (vector LDS reads)
  auto up4 = [](size_t v) { return (v + 3) / 4 * 4; };
  LdsLayout L;
  size_t o = 0;
  L.lut = o; o += (size_t)nsk * n_c * R;
  // the merge at the end reuses the LUT area: make sure it is large enough
  const size_t merge = (size_t)kWaves * R * (D + 2);
  if (o < merge) o = merge;
  o = up4(o);
  L.cv = o; o = up4(o + (size_t)n_c * dv);
  L.qt = o; o = up4(o + (size_t)R * D);
  L.pst = o; o = up4(o + (size_t)kWaves * 64 * R);
  L.vst = o; o = up4(o + (size_t)kWaves * 64 * nsv / 4);
  L.total_floats = o;
  return L;
}

template <int D, int R>
__global__ __launch_bounds__(kThreads) void attend_split_kernel(
    const __half* __restrict__ q, const uint8_t* __restrict__ kcodes,
    const float* __restrict__ kcb, const float* __restrict__ smooth,
    const uint8_t* __restrict__ vcodes, const float* __restrict__ vcb,
    const int32_t* __restrict__ kv_lens, float* __restrict__ part, const float* __restrict__ qpre,
    AttParams p) {
  extern __shared__ float smem[];
  const LdsLayout L = lds_layout(p.nsk, p.n_c, p.dv, p.nsv, R, D);
  float* lut = smem + L.lut;
  float* cv = smem + L.cv;
  float* qt = smem + L.qt;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  if (s_lo >= s_hi) {  // nothing to attend in this split
    if (tid < R) { out_part[tid * (D + 2)] = -INFINITY; out_part[tid * (D + 2) + 1] = 0.f; }
    return;
  }

  // ---- rows of this workgroup ------------------------------------------
  int qabs[R];
  bool rvalid[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int gr = rg * R + r;
    rvalid[r] = gr < p.rows;
    const int i = rvalid[r] ? gr % p.Sq : 0;
    qabs[r] = len - p.Sq + i;
  }

  // ---- dual transform of the queries: q~ = (q * s) . H ------------------
  const float* srow = smooth ? smooth + (size_t)(p.smooth_rows == 1 ? 0 : g) * D : nullptr;
  for (int idx = tid; idx < R * D; idx += kThreads) {
    const int r = idx / D, c = idx % D;
    const int gr = rg * R + r;
    float v = 0.f;
    if (gr < p.rows) {
      const int hl = gr / p.Sq, i = gr % p.Sq;
      const int h = g * p.G + hl;
      const size_t qi = (((size_t)b * p.Hq + h) * p.Sq + i) * D + c;
      if (qpre) {
        v = qpre[qi];  // dual-transformed already (explicit matrix)
      } else {
        v = __half2float(q[qi]);
        if (srow) v *= srow[c];
      }
    }
    qt[idx] = v;
  }
  __syncthreads();
  if (p.transform == 1) {
    for (int hb = 1; hb < D; hb <<= 1) {
      for (int k = tid; k < R * D / 2; k += kThreads) {
        const int r = k / (D / 2), m = k % (D / 2);
        const int i0 = (m / hb) * 2 * hb + (m % hb), i1 = i0 + hb;
        const float a = qt[r * D + i0], c = qt[r * D + i1];
        qt[r * D + i0] = a + c;
        qt[r * D + i1] = a - c;
      }
      __syncthreads();
    }
  }

  // ---- query LUT [j][code][row] and value codebook in LDS --------------
  for (int idx = tid; idx < p.nsk * p.n_c; idx += kThreads) {
    const int j = idx / p.n_c, c = idx % p.n_c;
    const float* crow = kcb + (size_t)c * p.dk;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    for (int e = 0; e < p.dk; ++e) {
      const float ce = crow[e];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = fmaf(qt[r * D + j * p.dk + e], ce, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] *= p.fold;
#pragma unroll
    for (int r = 0; r < R; ++r) lut[(size_t)idx * R + r] = acc[r];
  }
  for (int idx = tid; idx < p.n_c * p.dv; idx += kThreads) cv[idx] = vcb[idx];
  __syncthreads();

  // ---- stream the split's keys in 64-key chunks per wave ----------------
  constexpr int QPL = D / 4;          // 4-dim slices per head
  constexpr int TG = 64 / QPL;        // keys handled in parallel in the value phase
  const int dq = lane % QPL, ts = lane / QPL;
  float* pst = smem + L.pst + (size_t)wave * 64 * R;
  uint32_t* vst = reinterpret_cast<uint32_t*>(smem + L.vst) + (size_t)wave * 64 * (p.nsv / 4);
  const uint8_t* vst_b = reinterpret_cast<const uint8_t*>(vst);

  float m[R], l[R], acc[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY; l[r] = 0.f;
    acc[r][0] = acc[r][1] = acc[r][2] = acc[r][3] = 0.f;
  }

  const int n_tok = s_hi - s_lo;
  const int n_chunks = (n_tok + 63) / 64;
  const int n_iter = (n_chunks + kWaves - 1) / kWaves;
  const size_t row0 = (size_t)unit * p.S_cap;
  // bytes of a token's key / value code row; 32-bit words of codes
  const int cps = p.code_bits == 4 ? 2 : 1;  // codes per byte
  const int krow = p.nsk / cps, vrow = p.nsv / cps;
  const int nskw = krow / 4, nsvw = vrow / 4;
  const int cmax = p.n_c - 1;  // codes beyond the codebook are clamped, never read out of bounds

  for (int it = 0; it < n_iter; ++it) {
    const int chunk = it * kWaves + wave;
    const int t = s_lo + chunk * 64 + lane;
    const bool tv = chunk < n_chunks && t < s_hi;

    float sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) sc[r] = 0.f;
    if (tv) {
      const uint32_t* kr = reinterpret_cast<const uint32_t*>(kcodes + (row0 + t) * krow);
      if (p.code_bits == 4) {
        for (int jw = 0; jw < nskw; ++jw) {
          const uint32_t w = kr[jw];
#pragma unroll
          for (int k = 0; k < 8; ++k) {  // sub-vector 8 jw + k in nibble k
            const int code = min((int)((w >> (4 * k)) & 0xf), cmax);
            const float* e = lut + ((size_t)(jw * 8 + k) * p.n_c + code) * R;
            float v[R];
            lds_read_row<R>(e, v);
#pragma unroll
            for (int r = 0; r < R; ++r) sc[r] += v[r];
          }
        }
      } else {
        for (int jw = 0; jw < nskw; ++jw) {
          const uint32_t w = kr[jw];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int code = min((int)((w >> (8 * k)) & 0xff), cmax);
            const float* e = lut + ((size_t)(jw * 4 + k) * p.n_c + code) * R;
            float v[R];
            lds_read_row<R>(e, v);
#pragma unroll
            for (int r = 0; r < R; ++r) sc[r] += v[r];
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      bool ok = tv && rvalid[r];
      if (p.causal) ok = ok && t <= qabs[r];
      if (p.window > 0) ok = ok && t > qabs[r] - p.window;
      if (!ok) sc[r] = -INFINITY;
      const float cm = wave_max(sc[r]);
      const float mn = fmaxf(m[r], cm);
      const float alpha = (mn == -INFINITY) ? 1.f : exp2f(m[r] - mn);
      const float pr = (sc[r] == -INFINITY) ? 0.f : exp2f(sc[r] - mn);
      l[r] = l[r] * alpha + pr;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][e] *= alpha;
      m[r] = mn;
      pst[lane * R + r] = pr;
    }
    {
      const uint32_t* vr = reinterpret_cast<const uint32_t*>(vcodes + (row0 + (tv ? t : 0)) * vrow);
      for (int jw = 0; jw < nsvw; ++jw) vst[lane * nsvw + jw] = tv ? vr[jw] : 0u;
    }
    __syncthreads();

    for (int tt = 0; tt < 64 / TG; ++tt) {
      const int tk = tt * TG + ts;
      float pr[R];
      lds_read_row<R>(pst + tk * R, pr);
      const uint8_t* cr = vst_b + (size_t)tk * vrow;
      // code of value sub-vector i of this token
      auto vcode = [&](int i) {
        const int c = p.code_bits == 4 ? (cr[i >> 1] >> (4 * (i & 1))) & 15 : cr[i];
        return min(c, cmax);
      };
      float c4[4];
      if (p.dv >= 4) {
        const int dim0 = 4 * dq;
        const int code = vcode(dim0 / p.dv);
        const float4 v = *reinterpret_cast<const float4*>(cv + code * p.dv + dim0 % p.dv);
        c4[0] = v.x; c4[1] = v.y; c4[2] = v.z; c4[3] = v.w;
      } else if (p.dv == 2) {
        const int c0 = vcode(2 * dq), c1 = vcode(2 * dq + 1);
        c4[0] = cv[c0 * 2]; c4[1] = cv[c0 * 2 + 1];
        c4[2] = cv[c1 * 2]; c4[3] = cv[c1 * 2 + 1];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) c4[e] = cv[vcode(4 * dq + e)];
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(pr[r], c4[e], acc[r][e]);
    }
    __syncthreads();
  }

  // ---- merge lanes, then waves ------------------------------------------
#pragma unroll
  for (int r = 0; r < R; ++r) {
    l[r] = wave_sum(l[r]);
#pragma unroll
    for (int o = QPL; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][e] += __shfl_xor(acc[r][e], o);
  }
  float* wm = smem;                    // [kWaves][R]
  float* wl = wm + kWaves * R;         // [kWaves][R]
  float* wacc = wl + kWaves * R;       // [kWaves][R][D]
  // the LUT area is free once every wave has left the loop
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) { wm[wave * R + r] = m[r]; wl[wave * R + r] = l[r]; }
  }
  if (ts == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) wacc[((size_t)wave * R + r) * D + 4 * dq + e] = acc[r][e];
  }
  __syncthreads();
  for (int idx = tid; idx < R * (D + 2); idx += kThreads) {
    const int r = idx / (D + 2), c = idx % (D + 2);
    if (rg * R + r >= p.rows) continue;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w * R + r]);
    float v;
    if (c == 0) {
      v = M;
    } else {
      v = 0.f;
      for (int w = 0; w < kWaves; ++w) {
        const float mw = wm[w * R + r];
        const float om = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        v += om * (c == 1 ? wl[w * R + r] : wacc[((size_t)w * R + r) * D + (c - 2)]);
      }
    }
    out_part[idx] = v;
  }
}

// One block per output row: combine the splits with the log-sum-exp rule.
template <int D, int kRound>
__global__ __launch_bounds__(D) void attend_merge_kernel(const float* __restrict__ part,
                                                          __half* __restrict__ out, AttParams p) {
  const int row = blockIdx.x;  // ((b * Hq + h) * Sq + i)
  const int i = row % p.Sq;
  const int bh = row / p.Sq;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int g = h / p.G, hl = h % p.G;
  const int unit = b * p.Hkv + g;
  const int gr = hl * p.Sq + i;
  const int rg = gr / p.R, r = gr % p.R;
  const float* base = part + ((size_t)unit * p.n_rgroups + rg) * p.n_split * p.R * (D + 2) +
                      (size_t)r * (D + 2);
  const size_t stride = (size_t)p.R * (D + 2);
  // kRound splits per round: their (m, l) and the thread's accumulator value
  // are requested together (clamped addresses, masked values: no branch
  // between the loads), then folded into running sums rescaled to the
  // running max
  float M = -INFINITY, lsum = 0.f, a = 0.f;
  for (int s0 = 0; s0 < p.n_split; s0 += kRound) {
    float ms[kRound], ls[kRound], as[kRound];
#pragma unroll
    for (int k = 0; k < kRound; ++k) {
      const int sc = min(s0 + k, p.n_split - 1);
      const float* sp = base + sc * stride;
      ms[k] = sp[0];
      ls[k] = sp[1];
      as[k] = sp[2 + threadIdx.x];
    }
    // past the last split, or an empty split (its accumulator is not
    // written): weight zero, and the unwritten values never enter a product
#pragma unroll
    for (int k = 0; k < kRound; ++k) {
      if (s0 + k >= p.n_split) ms[k] = -INFINITY;
      if (ms[k] == -INFINITY) { ls[k] = 0.f; as[k] = 0.f; }
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < kRound; ++k) Mn = fmaxf(Mn, ms[k]);
    if (Mn == -INFINITY) continue;
    const float al = M == -INFINITY ? 0.f : exp2f(M - Mn);
    lsum *= al;
    a *= al;
#pragma unroll
    for (int k = 0; k < kRound; ++k) {
      const float w = ms[k] == -INFINITY ? 0.f : exp2f(ms[k] - Mn);
      lsum += w * ls[k];
      a += w * as[k];
    }
    M = Mn;
  }
  out[(size_t)row * D + threadIdx.x] = __float2half_rn(lsum > 0.f ? a / lsum : 0.f);
}

// Dual transform of every query row for an explicit matrix (transform 2):
// q~ = (q * s[kv(h)]) . (M^-1)^T in fp32, one workgroup per query row (the
// dual of the keys' x . M, "Metal Kernels API", "Fused SDPA": q~ . K~^T =
// q . K_hat^T).  Column j of (M^-1)^T is row j of M^-1.
__global__ __launch_bounds__(128) void dense_query_kernel(const __half* __restrict__ q,
                                                          const float* __restrict__ smooth,
                                                          const float* __restrict__ rot_inv,
                                                          float* __restrict__ out, int Hq, int Sq,
                                                          int D, int G, int smooth_rows) {
  extern __shared__ float xrow[];  // [D]
  const size_t row = blockIdx.x;   // (b, h, i)
  const int g = (int)((row / Sq) % Hq) / G;
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    float v = __half2float(q[row * D + i]);
    if (smooth) v *= smooth[(size_t)(smooth_rows == 1 ? 0 : g) * D + i];
    xrow[i] = v;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < D; j += blockDim.x) {
    const float* m = rot_inv + (size_t)j * D;
    float acc = 0.f;
    for (int i = 0; i < D; ++i) acc = fmaf(xrow[i], m[i], acc);
    out[row * D + j] = acc;
  }
}

template <int D, int R>
hipError_t launch_dr(const AttendArgs& a, const AttParams& p, size_t lds_bytes, hipStream_t st) {
  auto k = attend_split_kernel<D, R>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
  if (e != hipSuccess) return e;
  dim3 grid(a.B * a.Hkv, p.n_rgroups, p.n_split);
  hipLaunchKernelGGL(k, grid, dim3(kThreads), lds_bytes, st, a.q, a.k_codes, a.k_codebook,
                     a.smooth, a.v_codes, a.v_codebook, a.kv_lens, a.partials, a.q_pre, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attend_merge(a, p, st);
}

template <int D>
hipError_t launch_d(const AttendArgs& a, const AttParams& p, size_t lds_bytes, hipStream_t st) {
  switch (p.R) {
    case 1: return launch_dr<D, 1>(a, p, lds_bytes, st);
    case 2: return launch_dr<D, 2>(a, p, lds_bytes, st);
    case 4: return launch_dr<D, 4>(a, p, lds_bytes, st);
    case 8: return launch_dr<D, 8>(a, p, lds_bytes, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <int kRound>
hipError_t launch_merge_r(const AttendArgs& a, const AttParams& p, hipStream_t st) {
  const dim3 grid(a.B * a.Hq * a.Sq);
  switch (a.D) {
    case 32: hipLaunchKernelGGL((attend_merge_kernel<32, kRound>), grid, dim3(32), 0, st, a.partials, a.out, p); break;
    case 64: hipLaunchKernelGGL((attend_merge_kernel<64, kRound>), grid, dim3(64), 0, st, a.partials, a.out, p); break;
    case 128: hipLaunchKernelGGL((attend_merge_kernel<128, kRound>), grid, dim3(128), 0, st, a.partials, a.out, p); break;
    case 256: hipLaunchKernelGGL((attend_merge_kernel<256, kRound>), grid, dim3(256), 0, st, a.partials, a.out, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attend_merge(const AttendArgs& a, const AttParams& p, hipStream_t st) {
  // splits fetched per round: all of a short split list at once
  return p.n_split <= 4 ? launch_merge_r<4>(a, p, st) : launch_merge_r<16>(a, p, st);
}

// Key ranges up to this length run as one split per unit.
constexpr long long kOneSplitKeys = 1024;

bool plan_attend(int B, int Hq, int Sq, int D, int Hkv, int S_cap, int window, AttendPlan* pl) {
  if (B <= 0 || Hq <= 0 || Sq <= 0 || D <= 0 || Hkv <= 0 || S_cap <= 0 || window < 0) return false;
  if (Hq % Hkv != 0) return false;
  pl->G = Hq / Hkv;
  pl->rows = pl->G * Sq;
  const long long max_range =
      window > 0 ? std::min<long long>(S_cap, (long long)Sq + window - 1) : S_cap;
  // Aim for about 1024 workgroups (4 per CU on 256 CUs) across the
  // independent (batch row, kv head, 8-row group) units, with at least 512
  // keys per split so the per-workgroup LUT build stays amortized (256 and
  // 1024 measured slower on single-query decode at 2048 and 8192 keys).  Short
  // key ranges take one split: the per-unit kernel then writes the output
  // rows itself, and the merge launch it saves costs more than the longer
  // scan.
  const long long units = (long long)B * Hkv * ((pl->rows + 7) / 8);
  const long long target =
      max_range <= kOneSplitKeys ? 1 : std::max<long long>(1, (1024 + units - 1) / units);
  long long T = (max_range + target - 1) / target;
  T = (T + 63) / 64 * 64;
  T = std::max<long long>(T, 512);
  pl->split_tokens = (int)T;
  pl->n_split = (int)std::max<long long>(1, (max_range + T - 1) / T);
  const long long rows8 = (pl->rows + 7) / 8 * 8;
  pl->workspace_bytes = (size_t)B * Hkv * rows8 * pl->n_split * (D + 2) * sizeof(float);
  // the streaming kernel (chosen by the code sizes, which this call does not
  // see) may need more
  pl->workspace_bytes = std::max(pl->workspace_bytes, stream_workspace_bytes(B, Hq, Sq, D, Hkv));
  pl->workspace_bytes =
      std::max(pl->workspace_bytes, tile_workspace_bytes(B, Hq, Sq, D, Hkv, S_cap, window));
  // after the partials: the fp32 query rows of an explicit transform matrix
  pl->qpre_offset = (pl->workspace_bytes + 255) / 256 * 256;
  pl->workspace_bytes = pl->qpre_offset + (size_t)B * Hq * Sq * D * sizeof(float);
  pl->R = 0;
  pl->n_rgroups = 0;
  return true;
}

// LDS bytes of one workgroup for R rows; 0 if it does not fit.
static size_t attend_lds_bytes(int nsk, int n_c, int dv, int nsv, int R, int D) {
  const LdsLayout L = lds_layout(nsk, n_c, dv, nsv, R, D);
  const size_t bytes = L.total_floats * sizeof(float);
  return bytes <= kLdsBudget ? bytes : 0;
}

int attend_pick_rows(int rows, int nsk, int n_c, int dv, int nsv, int D, size_t* lds) {
  int want = 1;
  while (want < rows && want < 8) want <<= 1;
  for (int R = want; R >= 1; R >>= 1) {
    const size_t b = attend_lds_bytes(nsk, n_c, dv, nsv, R, D);
    if (b) { *lds = b; return R; }
  }
  return 0;
}

int attend_path(int B, int Hq, int Sq, int D, int Hkv, int S_cap, int window, int dk, int dv,
                int n_c, int code_bits, int transform) {
  // 4-bit codes and explicit transform matrices run on the streaming kernel
  // and the per-unit VALU kernel
  const bool basic = code_bits == 8 && transform != 2;
  if (basic && tile_plan(B, Hq, Sq, D, Hkv, S_cap, window, dk, dv, n_c, nullptr))
    return VQ_PATH_TILE;
  if (stream_plan(B, Hq, Sq, D, Hkv, S_cap, window, dk, dv, n_c, nullptr, nullptr, nullptr))
    return VQ_PATH_STREAM;
  AttendPlan plan;
  if (!plan_attend(B, Hq, Sq, D, Hkv, S_cap, window, &plan)) return 0;
  int R = 0;
  size_t lds = 0;
  if (basic && attend_mfma_plan(D, dv, D / dk, plan.rows, &R, &lds)) return VQ_PATH_LUT_MFMA;
  if (attend_pick_rows(plan.rows, D / dk, n_c, dv, D / dv, D, &lds)) return VQ_PATH_LUT_VALU;
  return 0;
}

hipError_t launch_attend(const AttendArgs& a_in, const AttendPlan& plan, hipStream_t st) {
  AttendArgs a = a_in;
  if (a.transform == 2) {
    // the query rows' dual transform, into the end of the workspace
    a.q_pre = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.partials) +
                                             plan.qpre_offset);
    const unsigned rows = (unsigned)((long long)a.B * a.Hq * a.Sq);
    hipLaunchKernelGGL(dense_query_kernel, dim3(rows), dim3(128), a.D * sizeof(float), st, a.q,
                       a.smooth, a.rot_inv, const_cast<float*>(a.q_pre), a.Hq, a.Sq, a.D,
                       a.Hq / a.Hkv, a.smooth_rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int path = attend_path(a.B, a.Hq, a.Sq, a.D, a.Hkv, a.S_cap, a.window, a.dk, a.dv, a.n_c,
                               a.code_bits, a.transform);
  if (path == VQ_PATH_TILE) {
    TileParams tp;
    tile_plan(a.B, a.Hq, a.Sq, a.D, a.Hkv, a.S_cap, a.window, a.dk, a.dv, a.n_c, &tp);
    return launch_attend_tile(a, tp, st);
  }
  if (path == VQ_PATH_STREAM) {
    StreamParams sp;
    size_t lds = 0;
    stream_plan(a.B, a.Hq, a.Sq, a.D, a.Hkv, a.S_cap, a.window, a.dk, a.dv, a.n_c, &sp, &lds, nullptr);
    return launch_attend_stream(a, sp, lds, st);
  }
  AttParams p;
  p.B = a.B; p.Hq = a.Hq; p.Sq = a.Sq; p.Hkv = a.Hkv; p.S_cap = a.S_cap;
  p.dk = a.dk; p.dv = a.dv; p.n_c = a.n_c; p.nsk = a.D / a.dk; p.nsv = a.D / a.dv;
  p.smooth_rows = a.smooth_rows; p.transform = a.transform; p.code_bits = a.code_bits;
  p.causal = a.causal; p.window = a.window;
  p.G = plan.G; p.rows = plan.rows; p.split_tokens = plan.split_tokens; p.n_split = plan.n_split;
  size_t lds = 0;
  const bool mfma = path == VQ_PATH_LUT_MFMA && attend_mfma_plan(a.D, a.dv, p.nsk, p.rows, &p.R, &lds);
  if (!mfma) p.R = attend_pick_rows(p.rows, p.nsk, p.n_c, p.dv, p.nsv, a.D, &lds);
  if (p.R == 0) return hipErrorInvalidValue;
  p.n_rgroups = (p.rows + p.R - 1) / p.R;
  if (p.n_rgroups > 65535 || p.n_split > 65535) return hipErrorInvalidValue;
  float norm = 1.f;
  if (a.transform == 1) {
    switch (a.D) {
      case 32: norm = WhtNorm<32>::value; break;
      case 64: norm = WhtNorm<64>::value; break;
      case 128: norm = WhtNorm<128>::value; break;
      case 256: norm = WhtNorm<256>::value; break;
    }
  }
  p.fold = norm * a.scale_log2e;
  if (mfma) return launch_attend_mfma(a, p, lds, st);
  switch (a.D) {
    case 32: return launch_d<32>(a, p, lds, st);
    case 64: return launch_d<64>(a, p, lds, st);
    case 128: return launch_d<128>(a, p, lds, st);
    case 256: return launch_d<256>(a, p, lds, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace vq
