// sep_mask_build kernels: separator flags, tile classes, dense mask.
//
// Visibility rule (SepLLM pages: P2 §1.2 mask matrix; P1 "SepAttention",
// build_prefill_mask): query i sees key j iff j <= i and (j < a, or
// i - j < n, or token j is a separator).
#include "common.hpp"
#include "internal.hpp"

namespace sep {

// One thread per 4 ids; the separator list is staged in LDS.
__global__ void __launch_bounds__(256) is_sep_kernel(const int32_t* __restrict__ ids, int64_t N,
                                                     const int32_t* __restrict__ sep_ids,
                                                     int n_sep, uint8_t* __restrict__ out) {
  __shared__ int32_t set[SEP_MAX_SEP_IDS_];
  for (int i = threadIdx.x; i < n_sep; i += blockDim.x) set[i] = sep_ids[i];
  __syncthreads();
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * 4;
  for (int64_t base = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; base < N;
       base += stride) {
    if (base + 4 <= N) {
      int4 v = *reinterpret_cast<const int4*>(ids + base);
      uchar4 o;
      o.x = in_set(v.x, set, n_sep);
      o.y = in_set(v.y, set, n_sep);
      o.z = in_set(v.z, set, n_sep);
      o.w = in_set(v.w, set, n_sep);
      *reinterpret_cast<uchar4*>(out + base) = o;
    } else {
      for (int64_t j = base; j < N; ++j) out[j] = in_set(ids[j], set, n_sep);
    }
  }
}

// One workgroup per (query tile qt, sequence b); each thread classifies the
// key tiles kt = threadIdx.x, threadIdx.x + blockDim.x, ...
//
// For queries [q0, q1) and keys [k0, k1), with V = "initial or separator"
// and NS = "neither":
//   class 0 if k0 > q1 - 1 (all keys in the future), or if k1 <= q0, no V
//           key in the block and k1 - 1 <= q0 - n (all keys past the window);
//   class 1 if k1 - 1 <= q0 and every NS key j has j >= q1 - n;
//   class 2 otherwise.
__global__ void __launch_bounds__(256) tile_class_kernel(const uint8_t* __restrict__ is_sep, int S,
                                                         int a, int n, int tq, int tk, int nkt,
                                                         uint8_t* __restrict__ tc) {
  const int qt = blockIdx.x;
  const int b = blockIdx.y;
  const uint8_t* f = is_sep + static_cast<int64_t>(b) * S;
  const int q0 = qt * tq;
  const int q1 = min(q0 + tq, S);
  uint8_t* row = tc + (static_cast<int64_t>(b) * gridDim.x + qt) * nkt;
  for (int kt = threadIdx.x; kt < nkt; kt += blockDim.x) {
    const int k0 = kt * tk;
    const int k1 = min(k0 + tk, S);
    uint8_t cls;
    if (k0 > q1 - 1) {
      cls = 0;
    } else {
      bool any_v = false;
      int min_ns = S;  // smallest NS key in the block
      for (int j = k0; j < k1; ++j) {
        const bool v = (j < a) || f[j];
        any_v |= v;
        if (!v && j < min_ns) min_ns = j;
      }
      if (k1 - 1 <= q0 && min_ns >= q1 - n) {
        cls = 1;
      } else if (k1 <= q0 && !any_v && (k1 - 1) <= q0 - n) {
        cls = 0;
      } else {
        cls = 2;
      }
    }
    row[kt] = cls;
  }
}

// One workgroup per (row i, sequence b); each thread writes 16 mask bytes.
__global__ void __launch_bounds__(256) dense_mask_kernel(const uint8_t* __restrict__ is_sep, int S,
                                                         int a, int n, uint8_t* __restrict__ M) {
  const int i = blockIdx.x;
  const int b = blockIdx.y;
  const uint8_t* f = is_sep + static_cast<int64_t>(b) * S;
  uint8_t* row = M + (static_cast<int64_t>(b) * S + i) * S;
  for (int j0 = threadIdx.x * 16; j0 < S; j0 += blockDim.x * 16) {
    uint8_t vals[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int j = j0 + e;
      bool vis = false;
      if (j < S && j <= i) vis = (j < a) || (i - j < n) || (f[j] != 0);
      vals[e] = vis;
    }
    if (j0 + 16 <= S && (S % 16) == 0) {
      uint4 pk;
      pk.x = vals[0] | (vals[1] << 8) | (vals[2] << 16) | (vals[3] << 24);
      pk.y = vals[4] | (vals[5] << 8) | (vals[6] << 16) | (vals[7] << 24);
      pk.z = vals[8] | (vals[9] << 8) | (vals[10] << 16) | (vals[11] << 24);
      pk.w = vals[12] | (vals[13] << 8) | (vals[14] << 16) | (vals[15] << 24);
      *reinterpret_cast<uint4*>(row + j0) = pk;
    } else {
      for (int e = 0; e < 16 && j0 + e < S; ++e) row[j0 + e] = vals[e];
    }
  }
}

hipError_t launch_is_sep(const int32_t* ids, int64_t N, const int32_t* sep_ids, int n_sep,
                         uint8_t* is_sep, hipStream_t st) {
  const int64_t groups = (N + 4 * 256 - 1) / (4 * 256);
  const int grid = static_cast<int>(groups < 8192 ? (groups > 0 ? groups : 1) : 8192);
  hipLaunchKernelGGL(is_sep_kernel, dim3(grid), dim3(256), 0, st, ids, N, sep_ids, n_sep, is_sep);
  return hipGetLastError();
}

hipError_t launch_tile_class(const uint8_t* is_sep, int B, int S, int a, int n, int tq, int tk,
                             uint8_t* tc, hipStream_t st) {
  const int nqt = (S + tq - 1) / tq;
  const int nkt = (S + tk - 1) / tk;
  hipLaunchKernelGGL(tile_class_kernel, dim3(nqt, B), dim3(256), 0, st, is_sep, S, a, n, tq, tk, nkt,
                     tc);
  return hipGetLastError();
}

hipError_t launch_dense_mask(const uint8_t* is_sep, int B, int S, int a, int n, uint8_t* M,
                             hipStream_t st) {
  hipLaunchKernelGGL(dense_mask_kernel, dim3(S, B), dim3(256), 0, st, is_sep, S, a, n, M);
  return hipGetLastError();
}

}  // namespace sep
