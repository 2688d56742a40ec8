// sep_attn_decode and sep_attn_decode_rope launches; the kernel body and its
// design are in decode.hpp (shared with the fused decode + update of
// cache.hip).
#include "decode.hpp"

namespace sep {

template <int D, int NW, bool ROPE>
__global__ void __launch_bounds__(NW * 64, ROPE ? 8 / NW : 1) decode_kernel(DecodeArgs A) {
  decode_body<D, NW, ROPE>(A, blockIdx.x, blockIdx.y, 0);
}

// Split decode, grid (Hkv * ns, B): range blockIdx.x % ns of the list of kv
// head blockIdx.x / ns, into its partial.
template <int D, bool ROPE>
__global__ void __launch_bounds__(kSplitWaves * 64) decode_split_kernel(DecodeArgs A) {
  decode_body<D, kSplitWaves, ROPE>(A, blockIdx.x / A.ns, blockIdx.y, blockIdx.x % A.ns);
}

// Merge of the partials, grid (Hkv, B).
template <int D>
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeArgs A) {
  merge_body<D>(A, blockIdx.x, blockIdx.y, 256);
}

template <int D, int NW>
static void launch_one(const DecodeArgs& A, int Hkv, int B, hipStream_t st) {
  if (A.rope != nullptr)
    hipLaunchKernelGGL((decode_kernel<D, NW, true>), dim3(Hkv, B), dim3(NW * kWave), 0, st, A);
  else
    hipLaunchKernelGGL((decode_kernel<D, NW, false>), dim3(Hkv, B), dim3(NW * kWave), 0, st, A);
}

template <int D>
static void launch_ranges(const DecodeArgs& A, int Hkv, int B, hipStream_t st) {
  const dim3 grid(Hkv * A.ns, B);
  if (A.rope != nullptr)
    hipLaunchKernelGGL((decode_split_kernel<D, true>), grid, dim3(kSplitWaves * kWave), 0, st, A);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, false>), grid, dim3(kSplitWaves * kWave), 0, st, A);
}

hipError_t launch_split_ranges(const DecodeArgs& A, const sep_cache& c, hipStream_t st) {
  if (c.D == 128) launch_ranges<128>(A, c.Hkv, c.B, st);
  else launch_ranges<64>(A, c.Hkv, c.B, st);
  return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k_new, const void* v_new, const sep_cache& c,
                         int Hq, float scale, const float* rope, void* out, float* lse, hipStream_t st) {
  const DecodeArgs A = decode_args(q, k_new, v_new, c, Hq, scale, rope, out, lse);
  if (A.part != nullptr) {
    const hipError_t e = launch_split_ranges(A, c, st);
    if (e != hipSuccess) return e;
    if (c.D == 128)
      hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(c.Hkv, c.B), dim3(256), 0, st, A);
    else
      hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(c.Hkv, c.B), dim3(256), 0, st, A);
    return hipGetLastError();
  }
  const bool wide = decode_uses_wide(c);
  if (c.D == 128) {
    if (wide) launch_one<128, 8>(A, c.Hkv, c.B, st);
    else launch_one<128, 4>(A, c.Hkv, c.B, st);
  } else {
    if (wide) launch_one<64, 8>(A, c.Hkv, c.B, st);
    else launch_one<64, 4>(A, c.Hkv, c.B, st);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- RoPE table
__global__ void rope_table_kernel(double base, int D, int n_pos, float* table) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int h = D / 2;
  if (e >= static_cast<int64_t>(n_pos) * h) return;
  const int p = static_cast<int>(e / h);
  const int i = static_cast<int>(e % h);
  const double ang = static_cast<double>(p) * pow(base, -2.0 * i / D);
  double sn, cs;
  sincos(ang, &sn, &cs);
  *reinterpret_cast<f32x2*>(table + 2 * e) = f32x2{static_cast<float>(cs), static_cast<float>(sn)};
}

hipError_t launch_rope_table(double base, int D, int n_pos, float* table, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(n_pos) * (D / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, base, D,
                     n_pos, table);
  return hipGetLastError();
}

}  // namespace sep
