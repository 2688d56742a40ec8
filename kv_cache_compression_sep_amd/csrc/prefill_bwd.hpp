// Shared pieces of the prefill backward kernels (prefill_bwd.hip: delta and
// the fp32 kernels; prefill_bwd_bf16.hip: the bf16 MFMA kernels, built with
// their own code-generation flag).
#pragma once

#include "prefill.hpp"
#include "internal.hpp"

namespace sep {
namespace bwd {

constexpr int BW = 4;                  // waves per workgroup
constexpr int BT = BW * kWave;
constexpr int KTQ = 64;                // keys per tile (dq_kernel)
constexpr int QB = 32;                 // query rows per tile (dk/dv kernels)
constexpr int KB = BW * 32;            // keys per dk/dv workgroup
constexpr int QCH = 256;               // query rows per dkdv_glob chunk
constexpr int kMaxChunks = SEP_MAX_BACKWARD_S / QCH;
static_assert(SEP_MAX_BACKWARD_S % QCH == 0, "whole chunks");

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  const uint8_t* is_sep;
  const int32_t* rank;
  const int32_t* sep_pos;
  float* delta;
  float* dq;
  float* dk;
  float* dv;
  int B, Hq, Hkv, S, a, n, G;
  float scale, scale_log2;
  // forward-style work items of dq_kernel
  int HPW, QT, n_hg, n_qt;
};

// Per-chunk tile counts of the global keys (ceil(n_global(chunk end) / KB))
// as an exclusive prefix in tstart[0 .. n_qc]; returns the total. Every one
// of the NT threads of the workgroup calls it (two barriers); wsum holds
// NT / 64 entries.
template <int NT = BT, class NGlobal>
__device__ int chunk_tile_prefix(NGlobal n_global, int S, int n_qc, int32_t* tstart, int32_t* wsum) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int seg = (n_qc + NT - 1) / NT;
  const int cb = min(tid * seg, n_qc);
  const int ce = min(cb + seg, n_qc);
  int local = 0;
  for (int c = cb; c < ce; ++c) {
    const int nt = (n_global(min((c + 1) * QCH, S)) + KB - 1) / KB;
    tstart[c] = nt;
    local += nt;
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += wsum[w];
  for (int c = cb; c < ce; ++c) {
    const int nt = tstart[c];
    tstart[c] = run;
    run += nt;
  }
  if (tid == NT - 1) tstart[n_qc] = run;          // the last thread's running sum is the total
  __syncthreads();
  return tstart[n_qc];
}

// Chunk of item w: the last c with tstart[c] <= w (it has tiles: w < tstart[c + 1]).
__device__ __forceinline__ int chunk_of(const int32_t* tstart, int n_qc, int w) {
  int lo = 0, hi = n_qc - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (tstart[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

hipError_t launch_bf16_kernels(const BwdArgs& A, int D, hipStream_t st);

}  // namespace bwd
}  // namespace sep
