// sep_attn_decode: one decode step over the four-block cache (GQA, bf16).
//
// The current token attends every retained entry (initial block, separator
// ring, recent ring) plus itself (SepLLM pages: P1 "Streaming-SepLLM", the
// step order is forward with the cache, then update; P1 "SepAttention",
// build_generate_mask applies the keep rule to one query; P2 §1.3, only the
// retained KV are read). The slot order does not matter for the result, so
// the retained entries are enumerated as a virtual list
//   u in [0, n_init)                 -> slot u
//   u in [n_init, n_init + cnt)      -> separator-ring slots
//   u in [.., occ)                   -> recent-ring slots of positions [rec_lo, t)
//   u == occ                         -> the new token (k_new / v_new)
//
// Grid (split, kv head, sequence): each workgroup takes one contiguous chunk
// of the virtual list for the G query heads of its kv head. Each wave owns a
// 32-key slice per iteration: S^T = K Q^T with the 16x16x32 bf16 MFMA (K rows
// read straight from HBM into the A operand, Q^T in registers), online
// softmax per head column, then O^T += V^T P^T with V staged transposed in
// the wave's own LDS slice. Waves merge through LDS; splits merge through
// the workspace, the last workgroup of a (sequence, kv head) to finish doing
// the final normalisation (ticket counter, reset to zero afterwards).
#include "common.hpp"
#include "internal.hpp"

namespace sep {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kSlice = 32;                       // keys per wave per iteration

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* kc;
  const uint16_t* vc;
  const int64_t* state;
  uint16_t* out;
  float* lse;
  float* part;       // [B*Hkv, nsplit, G*(D+2)]
  int* tickets;      // [B*Hkv]
  int a, s, p, w, c, Hq, Hkv, G, nsplit;
  float scale_log2;
};

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int c, int D) {
  (void)c;
  const int G = Hq / Hkv;
  const size_t rec = static_cast<size_t>(G) * (D + 2) * sizeof(float);
  size_t bytes = static_cast<size_t>(B) * Hkv * kDecodeMaxSplit * rec;
  bytes = (bytes + 255) & ~static_cast<size_t>(255);
  bytes += static_cast<size_t>(B) * Hkv * sizeof(int);
  return (bytes + 255) & ~static_cast<size_t>(255);
}

static inline size_t tickets_offset(int B, int Hkv, int G, int D) {
  const size_t rec = static_cast<size_t>(G) * (D + 2) * sizeof(float);
  size_t bytes = static_cast<size_t>(B) * Hkv * kDecodeMaxSplit * rec;
  return (bytes + 255) & ~static_cast<size_t>(255);
}

template <int D>
__global__ void __launch_bounds__(kDecThreads) decode_kernel(DecodeArgs A) {
  constexpr int VSTR = kSlice + 8;               // V^T row stride (bf16)
  constexpr int NDB = D / 16;                    // 16-row d-blocks of O^T
  constexpr int NKS = D / 32;                    // k-steps of QK^T
  __shared__ __attribute__((aligned(16))) uint16_t vt[kDecWaves][D * VSTR];
  __shared__ float red_m[kDecWaves][16];
  __shared__ float red_l[kDecWaves][16];
  __shared__ float red_o[kDecWaves][16][D + 1];
  __shared__ int last_flag;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int sp = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int G = A.G;
  const int rw = A.p + A.w;

  // ---- cache geometry of this sequence
  const int64_t* st = A.state + 4 * static_cast<int64_t>(b);
  const int64_t t = st[0];
  const int64_t K = st[1];
  const int head = static_cast<int>(st[2]);
  const int cnt = static_cast<int>(st[3]);
  const int n_init = static_cast<int>(t < A.a ? t : A.a);
  const int64_t cend = A.a + K * (A.p + 1);
  const int64_t rec_lo = cend > A.a ? cend : A.a;
  const int n_rec = static_cast<int>(t > rec_lo ? t - rec_lo : 0);
  const int occ = n_init + cnt + n_rec;
  const int L = occ + 1;
  const int chunk = (L + A.nsplit - 1) / A.nsplit;
  const int u_begin = sp * chunk;
  const int u_end = min(L, u_begin + chunk);

  const int64_t bg = static_cast<int64_t>(b) * A.Hkv + g;
  const uint16_t* kbase = A.kc + bg * A.c * D;
  const uint16_t* vbase = A.vc + bg * A.c * D;
  const uint16_t* knew = A.k_new + bg * D;
  const uint16_t* vnew = A.v_new + bg * D;

  // row pointer of virtual key u (clamped keys are masked later)
  auto row_of = [&](int u, const uint16_t* base, const uint16_t* nw) -> const uint16_t* {
    if (u >= occ) return nw;
    int slot;
    if (u < n_init) {
      slot = u;
    } else if (u < n_init + cnt) {
      int r = head - cnt + (u - n_init);
      r %= A.s;
      if (r < 0) r += A.s;
      slot = A.a + r;
    } else {
      const int64_t x = rec_lo + (u - n_init - cnt);
      slot = A.a + A.s + static_cast<int>((x - A.a) % rw);
    }
    return base + static_cast<int64_t>(slot) * D;
  };

  // ---- Q^T fragments: lane l holds head l%16 (zero beyond G),
  //      d = 32*ks + 8*(l/16) + i
  bf16x8 qf[NKS];
  {
    const int hq = lane % 16;
    const uint16_t* qrow = A.q + (static_cast<int64_t>(b) * A.Hq + g * G + (hq < G ? hq : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * (lane / 16));
      if (hq >= G) v = u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const int hh = lane / 16;

  const int span = u_end - u_begin;
  const int iters = span > 0 ? (span + kDecWaves * kSlice - 1) / (kDecWaves * kSlice) : 0;
  for (int it = 0; it < iters; ++it) {
    const int u0 = u_begin + (it * kDecWaves + wave) * kSlice;   // this wave's slice
    // ---- K fragments for two 16-key groups: lane row = key u0 + 16*gq + l%16
    bf16x8 kf[2][NKS];
#pragma unroll
    for (int gq = 0; gq < 2; ++gq) {
      const int u = u0 + 16 * gq + lane % 16;
      const uint16_t* kr = row_of(u < u_end ? u : u_begin, kbase, knew);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        kf[gq][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + 32 * ks + 8 * hh));
    }
    // ---- V rows -> transposed LDS slice. Pair index pi = (quad kq, chunk dc).
    //      Quads q (keys 4q..4q+3) go to column 8*(q%4) + 4*(q/4), so the
    //      eight keys a PV lane group needs ({4h..4h+3} and {16+4h..16+4h+3})
    //      are contiguous.
    constexpr int PAIRS = 8 * (D / 8);
#pragma unroll
    for (int pi0 = 0; pi0 < PAIRS; pi0 += kWave) {
      const int pi = pi0 + lane;
      const int kq = pi % 8;
      const int dc = pi / 8;
      u32x4 vr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int u = u0 + 4 * kq + e;
        const uint16_t* vrp = row_of(u < u_end ? u : u_begin, vbase, vnew);
        vr[e] = *reinterpret_cast<const u32x4*>(vrp + 8 * dc);
      }
      const int col = 8 * (kq % 4) + 4 * (kq / 4);
      uint16_t* V = vt[wave];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t w01e = __builtin_amdgcn_perm(vr[1][m], vr[0][m], 0x05040100u);
        const uint32_t w23e = __builtin_amdgcn_perm(vr[3][m], vr[2][m], 0x05040100u);
        const uint32_t w01o = __builtin_amdgcn_perm(vr[1][m], vr[0][m], 0x07060302u);
        const uint32_t w23o = __builtin_amdgcn_perm(vr[3][m], vr[2][m], 0x07060302u);
        const int d = 8 * dc + 2 * m;
        *reinterpret_cast<u32x2*>(V + d * VSTR + col) = u32x2{w01e, w23e};
        *reinterpret_cast<u32x2*>(V + (d + 1) * VSTR + col) = u32x2{w01o, w23o};
      }
    }
    // ---- scores S^T: lane l holds head l%16, keys 16*gq + 4*(l/16) + r
    f32x4 s[2];
#pragma unroll
    for (int gq = 0; gq < 2; ++gq) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc = mfma16x16x32(kf[gq][ks], qf[ks], acc);
      s[gq] = acc;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int gq = 0; gq < 2; ++gq)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = u0 + 16 * gq + 4 * hh + r;
        if (u >= u_end) s[gq][r] = -INFINITY;
        mx = fmaxf(mx, s[gq][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * A.scale_log2;
    const float m_new = fmaxf(m_run, mx);
    const float corr = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
    m_run = m_new;
    const float msub = (m_new == -INFINITY) ? 0.0f : m_new;
    float lsum = 0.f;
    u32x4 pk;
#pragma unroll
    for (int gq = 0; gq < 2; ++gq) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[gq][r] = fast_exp2(__builtin_fmaf(s[gq][r], A.scale_log2, -msub));
        lsum += s[gq][r];
      }
      pk[2 * gq] = pack_bf16x2(s[gq][0], s[gq][1]);
      pk[2 * gq + 1] = pack_bf16x2(s[gq][2], s[gq][3]);
    }
    l_run = l_run * corr + lsum;
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
    __syncthreads();  // V^T slices written
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint16_t* vrow = vt[wave] + (16 * db + lane % 16) * VSTR + 8 * hh;
      const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vrow));
      oacc[db] = oacc[db] * corr;
      oacc[db] = mfma16x16x32(av, pb, oacc[db]);
    }
    __syncthreads();  // V^T slices consumed
  }

  // ---- merge the waves: lane l holds head l%16, d = 16*db + 4*(l/16) + r;
  //      l_run is a partial sum over this lane group's keys.
  float lw = l_run;
  lw += __shfl_xor(lw, 16, kWave);
  lw += __shfl_xor(lw, 32, kWave);
  if (lane < 16) {
    red_m[wave][lane] = m_run;
    red_l[wave][lane] = lw;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) red_o[wave][lane % 16][16 * db + 4 * hh + r] = oacc[db][r];
  __syncthreads();

  // thread e handles (head, d) pairs of this workgroup's merged partial
  const int rec = G * (D + 2);
  float* part = A.part + (bg * A.nsplit + sp) * rec;
  for (int e = tid; e < G * D; e += kDecThreads) {
    const int hq = e / D;
    const int d = e % D;
    float M = -INFINITY;
    for (int wv = 0; wv < kDecWaves; ++wv) M = fmaxf(M, red_m[wv][hq]);
    float o = 0.f, l = 0.f;
    for (int wv = 0; wv < kDecWaves; ++wv) {
      const float f = (red_m[wv][hq] == -INFINITY) ? 0.f : fast_exp2(red_m[wv][hq] - M);
      o += f * red_o[wv][hq][d];
      l += f * red_l[wv][hq];
    }
    part[hq * (D + 2) + d] = o;
    if (d == 0) {
      part[hq * (D + 2) + D] = M;
      part[hq * (D + 2) + D + 1] = l;
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int prev = atomicAdd(&A.tickets[bg], 1);
    last_flag = (prev == A.nsplit - 1);
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  const float* parts = A.part + bg * A.nsplit * rec;
  for (int e = tid; e < G * D; e += kDecThreads) {
    const int hq = e / D;
    const int d = e % D;
    float M = -INFINITY;
    for (int j = 0; j < A.nsplit; ++j) M = fmaxf(M, __builtin_nontemporal_load(parts + j * rec + hq * (D + 2) + D));
    float o = 0.f, l = 0.f;
    for (int j = 0; j < A.nsplit; ++j) {
      const float* pr = parts + j * rec + hq * (D + 2);
      const float mj = __builtin_nontemporal_load(pr + D);
      const float f = (mj == -INFINITY) ? 0.f : fast_exp2(mj - M);
      o += f * __builtin_nontemporal_load(pr + d);
      l += f * __builtin_nontemporal_load(pr + D + 1);
    }
    const int64_t orow = static_cast<int64_t>(b) * A.Hq + g * G + hq;
    const float val = o / l;
    const uint32_t bits = pack_bf16x2(val, 0.f);
    A.out[orow * D + d] = static_cast<uint16_t>(bits & 0xffffu);
    if (d == 0 && A.lse != nullptr) A.lse[orow] = (M + fast_log2(l)) * kLn2;
  }
  if (tid == 0) A.tickets[bg] = 0;
}

hipError_t launch_decode(const void* q, const void* k_new, const void* v_new, const sep_cache& c,
                         int Hq, float scale, void* out, float* lse, void* ws, hipStream_t st) {
  DecodeArgs A;
  A.q = static_cast<const uint16_t*>(q);
  A.k_new = static_cast<const uint16_t*>(k_new);
  A.v_new = static_cast<const uint16_t*>(v_new);
  A.kc = static_cast<const uint16_t*>(c.k);
  A.vc = static_cast<const uint16_t*>(c.v);
  A.state = c.state;
  A.out = static_cast<uint16_t*>(out);
  A.lse = lse;
  A.a = c.a;
  A.s = c.s;  // the separator-ring branch is only reached when cnt > 0, i.e. s >= 1
  A.p = c.p;
  A.w = c.w;
  A.c = c.a + c.s + c.p + c.w;
  A.Hq = Hq;
  A.Hkv = c.Hkv;
  A.G = Hq / c.Hkv;
  const int pairs = c.B * c.Hkv;
  int ns = (2048 + pairs - 1) / pairs;
  const int max_by_len = (A.c + 1 + kSlice - 1) / kSlice;
  if (ns > max_by_len) ns = max_by_len;
  if (ns > kDecodeMaxSplit) ns = kDecodeMaxSplit;
  if (ns < 1) ns = 1;
  A.nsplit = ns;
  A.part = static_cast<float*>(ws);
  A.tickets = reinterpret_cast<int*>(static_cast<char*>(ws) + tickets_offset(c.B, c.Hkv, A.G, c.D));
  A.scale_log2 = scale * kLog2e;
  if (c.D == 128)
    hipLaunchKernelGGL(decode_kernel<128>, dim3(ns, c.Hkv, c.B), dim3(kDecThreads), 0, st, A);
  else
    hipLaunchKernelGGL(decode_kernel<64>, dim3(ns, c.Hkv, c.B), dim3(kDecThreads), 0, st, A);
  return hipGetLastError();
}

}  // namespace sep
