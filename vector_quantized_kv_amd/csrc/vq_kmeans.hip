// Codebook training for gfx950: Lloyd's k-means over pooled sub-vectors.
//
// Method: the codebooks of the "veloxquant_mlx.cache.vecinfer_cache module"
// page come pre-trained (module description: keys are encoded against a
// pre-trained codebook).  The training taken here is Lloyd's algorithm on the
// sub-vectors the encode sees: every vector goes to its nearest centroid
// (fp32 squared distance summed over the sub-vector in index order, lowest
// index on exact ties: the per-lane encode kernels' search, so a trained
// codebook and the encode agree on what "nearest" means), then every
// centroid moves to the mean of its members; a centroid with no member keeps
// its value.
//
// One iteration is two launches on the caller's stream, with no host
// synchronization between iterations:
//   assign  sub-vectors of 8, from 65,536 of them: the encode's matrix-core
//           search (kmeans_f16_kernel in the encode source) with the same
//           accumulation as below.  Otherwise:
//           at most one 16-wave workgroup per CU.  A lane takes one vector at
//           a time (grid-stride), walks the codebook with a wave-uniform
//           centroid index (scalar loads shared by the 64 lanes), and adds
//           the vector, a count and its smallest distance into fp64
//           accumulators in LDS (LDS atomics).  The workgroup then writes its
//           accumulators to its own row of the workspace, every slot, so
//           nothing has to be cleared between iterations.
//   update  one workgroup per centroid, plus one for the inertia, sums its
//           slots over the workspace rows in a fixed order in fp64, divides
//           and rounds the mean to fp32 in place.
// Work per iteration: N * n_c * sub_dim subtract / multiply-add pairs on the
// vector ALUs; the N * sub_dim * 4 bytes read are small beside it.
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kAssignThreads = 1024;  // 16 waves
constexpr int kUpdateThreads = 256;
// From this many vectors of 8 the assignment runs on the matrix cores (the
// encode's split-fp16 search); below it the direct fp32 search, whose
// decisions match the per-lane encode exactly.
constexpr long long kMatrixMin = 65536;

template <int DS>
__device__ __forceinline__ void load_vec(const float* __restrict__ p, float (&x)[DS]) {
  if constexpr (DS == 1) {
    x[0] = p[0];
  } else if constexpr (DS == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    x[0] = v.x; x[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < DS; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(p + i);
      x[i] = v.x; x[i + 1] = v.y; x[i + 2] = v.z; x[i + 3] = v.w;
    }
  }
}

// Accumulator slots of one workgroup: centroid c owns [c * (DS + 1), ...):
// DS coordinate sums then the member count; slot n_c * (DS + 1) holds the
// sum of the smallest distances (the inertia).
template <int DS>
__global__ __launch_bounds__(kAssignThreads) void kmeans_assign_kernel(
    const float* __restrict__ x, long long N, const float* __restrict__ cb, int n_c,
    double* __restrict__ partials, uint8_t* __restrict__ labels) {
  constexpr int W = DS + 1;
  __shared__ double acc[256 * W + 1];
  const int slots = n_c * W + 1;
  for (int i = threadIdx.x; i < slots; i += kAssignThreads) acc[i] = 0.0;
  __syncthreads();

  double inert = 0.0;
  const long long stride = (long long)gridDim.x * kAssignThreads;
  // the trip count is the same for the whole workgroup; lanes past N search
  // vector 0 and discard the result
  for (long long base = (long long)blockIdx.x * kAssignThreads; base < N; base += stride) {
    const long long i = base + threadIdx.x;
    const bool ok = i < N;
    float v[DS];
    load_vec<DS>(x + (ok ? i : 0) * DS, v);
    float best = INFINITY;
    int idx = 0;
#pragma unroll 8
    for (int c = 0; c < n_c; ++c) {
      const float* cc = cb + c * DS;
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) {
        const float df = v[e] - cc[e];
        a = fmaf(df, df, a);
      }
      if (a < best) { best = a; idx = c; }
    }
    if (ok) {
      double* slot = acc + idx * W;
#pragma unroll
      for (int e = 0; e < DS; ++e) atomicAdd(slot + e, (double)v[e]);
      atomicAdd(slot + DS, 1.0);
      inert += (double)best;
      if (labels) labels[i] = (uint8_t)idx;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) inert += __shfl_xor(inert, m);
  if ((threadIdx.x & 63) == 0) atomicAdd(acc + n_c * W, inert);
  __syncthreads();
  double* row = partials + (size_t)blockIdx.x * slots;
  for (int i = threadIdx.x; i < slots; i += kAssignThreads) row[i] = acc[i];
}

template <int DS>
__global__ __launch_bounds__(kUpdateThreads) void kmeans_update_kernel(
    const double* __restrict__ partials, int G, int n_c, float* __restrict__ cb,
    double* __restrict__ inertia) {
  constexpr int W = DS + 1;
  constexpr int kWaves = kUpdateThreads / 64;
  const int slots = n_c * W + 1;
  const int c = blockIdx.x;  // c == n_c: the inertia slot
  const int first = c < n_c ? c * W : n_c * W;
  const int n = c < n_c ? W : 1;
  double s[W];
#pragma unroll
  for (int k = 0; k < W; ++k) s[k] = 0.0;
  for (int g = threadIdx.x; g < G; g += kUpdateThreads) {
    const double* row = partials + (size_t)g * slots + first;
#pragma unroll
    for (int k = 0; k < W; ++k)
      if (k < n) s[k] += row[k];
  }
  // fixed-order sum over the workgroup: butterflies in each wave, then the
  // wave totals in wave order
  __shared__ double red[kWaves][W];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    double t = s[k];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) t += __shfl_xor(t, m);
    s[k] = t;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int k = 0; k < W; ++k) red[wave][k] = s[k];
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  double tot[W];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    double t = red[0][k];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += red[w][k];
    tot[k] = t;
  }
  if (c < n_c) {
    if (tot[DS] > 0.0) {
#pragma unroll
      for (int e = 0; e < DS; ++e) cb[c * DS + e] = (float)(tot[e] / tot[DS]);
    }
  } else if (inertia) {
    *inertia = tot[0];
  }
}

template <int DS>
hipError_t run_kmeans(const KmeansArgs& a, hipStream_t st) {
  const int G = kmeans_blocks(a.N);
  for (int it = 0; it < a.iters; ++it) {
    uint8_t* labels = it + 1 == a.iters ? a.labels : nullptr;
    if (DS == 8 && a.N >= kMatrixMin) {
      const hipError_t e = launch_kmeans_assign_f16(a.vectors, a.N, a.centroids, a.n_c, a.partials, G,
                                                    labels, st);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(kmeans_assign_kernel<DS>, dim3(G), dim3(kAssignThreads), 0, st, a.vectors,
                         a.N, a.centroids, a.n_c, a.partials, labels);
    }
    hipLaunchKernelGGL(kmeans_update_kernel<DS>, dim3(a.n_c + 1), dim3(kUpdateThreads), 0, st,
                       a.partials, G, a.n_c, a.centroids, a.inertia ? a.inertia + it : nullptr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

int kmeans_blocks(long long N) {
  // at least four vectors per lane before a second workgroup, at most one
  // workgroup per CU of the 256
  const long long per = 4LL * kAssignThreads;
  const long long g = (N + per - 1) / per;
  return (int)(g < 1 ? 1 : (g > 256 ? 256 : g));
}

size_t kmeans_workspace_bytes(long long N, int sub_dim, int n_c) {
  return (size_t)kmeans_blocks(N) * (size_t)(n_c * (sub_dim + 1) + 1) * sizeof(double);
}

hipError_t launch_kmeans(const KmeansArgs& a, hipStream_t st) {
  switch (a.sub_dim) {
    case 1: return run_kmeans<1>(a, st);
    case 2: return run_kmeans<2>(a, st);
    case 4: return run_kmeans<4>(a, st);
    case 8: return run_kmeans<8>(a, st);
    case 16: return run_kmeans<16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace vq
