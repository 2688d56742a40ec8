// sep_attn_decode: one decode step over the four-block cache (GQA, bf16).
//
// The current token attends every retained entry (initial block, separator
// ring, recent ring) plus itself (SepLLM pages: P1 "Streaming-SepLLM", the
// step order is forward with the cache, then update; P1 "SepAttention",
// build_generate_mask applies the keep rule to one query; P2 §1.3, only the
// retained KV are read). The slot order does not matter for the result, so
// the retained entries are enumerated as a virtual list
//   u in [0, n_init)                 -> slot u
//   u in [n_init, n_init + cnt)      -> separator-ring slots, oldest first
//   u in [.., occ)                   -> recent-ring slots of positions [rec_lo, t)
//   u == occ                         -> the new token (k_new / v_new)
//
// One workgroup per (kv head, sequence) reads that list once; or, when the
// cache carries a work buffer and there are few (sequence, kv head) pairs,
// ns workgroups per pair each read one range of `span` consecutive entries
// of the list, every wave writing its unnormalised partial (running max, sum
// of weights, weighted sum of values, per query head) straight from its
// registers to the work buffer, and a second kernel merges the partials
// with the log-sum-exp rule (the
// kernel boundary orders the two; merging inside one kernel would need a
// device-scope release and acquire per workgroup, which on this GPU write
// back and invalidate the L2 of each XCD). Waves take 32-key slices, NW slices per iteration: S^T = K Q^T
// with the 16x16x32 bf16 MFMA (K rows loaded straight into the A operand,
// Q^T of the G query heads in registers), online softmax per head column,
// then O^T += V^T P^T with V staged transposed in the wave's own LDS slice
// (so the waves need no barrier until they merge). The next slice's K and V
// rows are loaded while the current one is computed. Waves merge through LDS
// at the end.
//
// With ROPE (sep_attn_decode_rope; P1 "Streaming-SepLLM": streaming needs
// positional-encoding shifting; RoFormer §3.4 for the rotation), virtual
// key u is exactly its shifted position: the cache holds unrotated keys and
// key u is rotated by u theta_i when its slice is consumed, the query by
// occ theta_i once; pair i is (x_i, x_{i+D/2}), which a lane holds in k-steps
// ks and ks + NKS/2 of the same fragment, so the rotation is lane-local. A
// lane's keys advance by 32 NW positions per slice, so their angles advance
// by one complex product per slice instead of a table load per key.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace sep {

constexpr int kSlice = 32;  // keys per wave per iteration

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* kc;
  const uint16_t* vc;
  const int64_t* state;
  uint16_t* out;
  float* lse;
  const float* rope;                             // [n_pos][D/2] (cos, sin), ROPE only
  float* part;                                   // split mode: partials [B][Hkv][np][G][part_stride]; else null
  int a, s, p, w, rw, c, Hq, Hkv, G;
  int ns, span, np;                              // split mode: ranges per list, entries per range, partials per list
  float scale_log2;
};

// One partial: running max (log2 domain), sum of weights, two pad words, then
// the weighted sum of values over d (16-byte aligned rows).
template <int D>
constexpr int part_stride() { return D + 4; }

__device__ __forceinline__ float bf16lo_f(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi_f(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Rotate the pairs (lo[e], hi[e]) of two bf16x8 fragments by the angles
// whose (cos, sin) are cs[e] (as four f32x4 of two pairs each); results are
// rounded to bf16.
__device__ __forceinline__ void rotate_pairs(u32x4& lo, u32x4& hi, const f32x4 (&cs)[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {                  // bf16 elements 2m, 2m + 1
    const float x0 = bf16lo_f(lo[m]), x1 = bf16hi_f(lo[m]);
    const float y0 = bf16lo_f(hi[m]), y1 = bf16hi_f(hi[m]);
    const float c0 = cs[m][0], s0 = cs[m][1], c1 = cs[m][2], s1 = cs[m][3];
    lo[m] = pack_bf16x2(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
    hi[m] = pack_bf16x2(y0 * c0 + x0 * s0, y1 * c1 + x1 * s1);
  }
}

// Decode of kv head g of sequence b: the whole list (A.part null) into out /
// lse, or range `split` of it into its partial.
template <int D, int NW, bool ROPE>
__device__ __forceinline__ void decode_body(const DecodeArgs& A, int g, int b, int split) {
  constexpr int NT = NW * kWave;
  constexpr int VSTR = kSlice + 8;               // V^T row stride (bf16)
  constexpr int NDB = D / 16;                    // 16-row d-blocks of O^T
  constexpr int NKS = D / 32;                    // k-steps of QK^T
  constexpr int PAIRS = 8 * (D / 8);             // (key quad, 16-byte chunk) pairs per slice
  constexpr int NPAIR = PAIRS / kWave;
  constexpr int VT_BYTES = NW * D * VSTR * 2;
  constexpr int RED_BYTES = NW * 16 * (D + 1) * 4;
  constexpr int ARENA = VT_BYTES > RED_BYTES ? VT_BYTES : RED_BYTES;
  constexpr int STEP_BYTES = ROPE ? 2 * 4 * (NKS / 2) * 4 * 16 : 0;   // RoPE angle steps, after the arena
  __shared__ __attribute__((aligned(16))) char arena[ARENA + STEP_BYTES];
  __shared__ float red_m[NW][16];
  __shared__ float red_l[NW][16];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int G = A.G;
  const int rw = A.rw;                          // recent-ring size
  uint16_t* vt = reinterpret_cast<uint16_t*>(arena) + wave * (D * VSTR);

  // ---- cache geometry of this sequence (wave-uniform scalars)
  const int64_t* st = A.state + kStateWords * static_cast<int64_t>(b);
  const int64_t t = st[0];
  const int64_t ncomp = st[1];                   // entries compacted out of R so far
  const int head = static_cast<int>(st[2]);
  const int cnt = static_cast<int>(st[3]);
  const int n_init = static_cast<int>(t < A.a ? t : A.a);
  const int64_t cend = A.a + ncomp;
  const int64_t rec_lo = cend > A.a ? cend : A.a;
  const int n_rec = static_cast<int>(t > rec_lo ? t - rec_lo : 0);
  const int u_s = n_init;                        // first separator-ring entry
  const int u_r = n_init + cnt;                  // first recent-ring entry
  const int occ = u_r + n_rec;
  const int L = occ + 1;
  // the entries [ub, ue) this workgroup reads (all of them without a split)
  const int ub = A.part == nullptr ? 0 : split * A.span;
  const int ue = A.part == nullptr ? L : min(L, ub + A.span);
  int s0 = 0;                                    // ring index of the oldest separator
  if (cnt > 0) {
    s0 = (head - cnt) % A.s;
    if (s0 < 0) s0 += A.s;
  }
  const int r0 = n_rec > 0 ? static_cast<int>((rec_lo - A.a) % rw) : 0;

  const int64_t bg = static_cast<int64_t>(b) * A.Hkv + g;
  const uint16_t* kbase = A.kc + bg * A.c * D;
  const uint16_t* vbase = A.vc + bg * A.c * D;
  const uint16_t* knew = A.k_new + bg * D;
  const uint16_t* vnew = A.v_new + bg * D;

  // slot of virtual key u (u < occ); keys past the list are clamped by callers
  auto slot_of = [&](int u) -> int {
    if (u < u_s) return u;
    if (u < u_r) {
      int r = s0 + (u - u_s);
      r = r >= A.s ? r - A.s : r;
      return A.a + r;
    }
    int r = r0 + (u - u_r);
    r = r >= rw ? r - rw : r;
    return A.a + A.s + r;
  };
  auto row_ptr = [&](int u, const uint16_t* base, const uint16_t* nw) -> const uint16_t* {
    if (u >= occ) return nw;
    return base + static_cast<int64_t>(slot_of(u)) * D;
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

  // ---- per-slice loads into registers
  struct Regs {
    u32x4 k[2][NKS];
    u32x4 v[NPAIR][4];
  };
  auto load_slice = [&](int u0, Regs& R) {
#pragma unroll
    for (int gq = 0; gq < 2; ++gq) {
      const int u = min(u0 + 16 * gq + lane % 16, ue - 1);
      const uint16_t* kr = row_ptr(u, kbase, knew);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        R.k[gq][ks] = *reinterpret_cast<const u32x4*>(kr + 32 * ks + 8 * hh);
    }
#pragma unroll
    for (int j = 0; j < NPAIR; ++j) {
      const int pi = j * kWave + lane;
      const int kq = pi % 8;
      const int dc = pi / 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int u = min(u0 + 4 * kq + e, ue - 1);
        R.v[j][e] = *reinterpret_cast<const u32x4*>(row_ptr(u, vbase, vnew) + 8 * dc);
      }
    }
  };

  const int iters = ue > ub ? (ue - ub + NW * kSlice - 1) / (NW * kSlice) : 0;
  // ROPE: (cos, sin) of this lane's pairs at its first key of the current
  // slice, u = (it NW + wave) 32 + lane % 16; its second key (u + 16) takes
  // one complex product with the angles of 16 positions. Between slices u
  // grows by 32 NW, so the angles advance by one complex product with that
  // row of the table; every 16th slice they are reloaded from the table,
  // which keeps the fp32 drift of the products to a few ulp. The two step
  // rows depend on the lane only through lane / 16 and sit in LDS.
  f32x4 rc[ROPE ? NKS / 2 : 1][4];
  // [16 | 32 NW][lane / 16][ks][m]
  auto rstep = reinterpret_cast<f32x4(*)[4][NKS / 2 > 0 ? NKS / 2 : 1][4]>(arena + ARENA);
  auto load_angles = [&](int it) {
    const int u = min(ub + (it * NW + wave) * kSlice + lane % 16, L - 1);
    const float* trow = A.rope + static_cast<int64_t>(u) * D;
#pragma unroll
    for (int ks = 0; ks < NKS / 2; ++ks)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        rc[ks][m] = *reinterpret_cast<const f32x4*>(trow + 2 * (32 * ks + 8 * hh + 2 * m));
  };
  auto cmul = [](f32x4 a, f32x4 d) {
    return f32x4{a[0] * d[0] - a[1] * d[1], a[1] * d[0] + a[0] * d[1], a[2] * d[2] - a[3] * d[3],
                 a[3] * d[2] + a[2] * d[3]};
  };
  Regs cur;
  if (iters > 0) load_slice(ub + wave * kSlice, cur);   // the first slice's K/V in flight before the table reads
  if constexpr (ROPE) {
    {                                            // the query at position occ
      const float* trow = A.rope + static_cast<int64_t>(occ) * D;
#pragma unroll
      for (int ks = 0; ks < NKS / 2; ++ks) {
        f32x4 cs[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          cs[m] = *reinterpret_cast<const f32x4*>(trow + 2 * (32 * ks + 8 * hh + 2 * m));
        u32x4 lo = __builtin_bit_cast(u32x4, qf[ks]), hi = __builtin_bit_cast(u32x4, qf[ks + NKS / 2]);
        rotate_pairs(lo, hi, cs);
        qf[ks] = __builtin_bit_cast(bf16x8, lo);
        qf[ks + NKS / 2] = __builtin_bit_cast(bf16x8, hi);
      }
    }
    load_angles(0);
    constexpr int NST = 4 * (NKS / 2) * 4;
    if (tid < 2 * NST) {
      const int which = tid / NST, e = tid % NST;
      const int h4 = e / ((NKS / 2) * 4), ks = (e / 4) % (NKS / 2), m = e % 4;
      // row 16 exists when L > 16, row 32 NW when L > 32 NW; otherwise the
      // keys that would use them are past the list and masked
      const int row = which == 0 ? 16 : NW * kSlice;
      f32x4 v = f32x4{1.f, 0.f, 1.f, 0.f};
      if (L > row) v = *reinterpret_cast<const f32x4*>(A.rope + static_cast<int64_t>(row) * D +
                                                         2 * (32 * ks + 8 * h4 + 2 * m));
      rstep[which][h4][ks][m] = v;
    }
    __syncthreads();
  }
  for (int it = 0; it < iters; ++it) {
    const int u0 = ub + (it * NW + wave) * kSlice;   // this wave's slice
    // ---- V rows -> transposed LDS slice. Quads q (keys 4q..4q+3) go to
    //      column 8*(q%4) + 4*(q/4), so the eight keys a PV lane group needs
    //      ({4h..4h+3} and {16+4h..16+4h+3}) are contiguous.
#pragma unroll
    for (int j = 0; j < NPAIR; ++j) {
      const int pi = j * kWave + lane;
      const int kq = pi % 8;
      const int dc = pi / 8;
      const int col = 8 * (kq % 4) + 4 * (kq / 4);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t w01e = __builtin_amdgcn_perm(cur.v[j][1][m], cur.v[j][0][m], 0x05040100u);
        const uint32_t w23e = __builtin_amdgcn_perm(cur.v[j][3][m], cur.v[j][2][m], 0x05040100u);
        const uint32_t w01o = __builtin_amdgcn_perm(cur.v[j][1][m], cur.v[j][0][m], 0x07060302u);
        const uint32_t w23o = __builtin_amdgcn_perm(cur.v[j][3][m], cur.v[j][2][m], 0x07060302u);
        const int d = 8 * dc + 2 * m;
        *reinterpret_cast<u32x2*>(vt + d * VSTR + col) = u32x2{w01e, w23e};
        *reinterpret_cast<u32x2*>(vt + (d + 1) * VSTR + col) = u32x2{w01o, w23o};
      }
    }
    if constexpr (ROPE) {
#pragma unroll
      for (int ks = 0; ks < NKS / 2; ++ks) {
        rotate_pairs(cur.k[0][ks], cur.k[0][ks + NKS / 2], rc[ks]);
        f32x4 c16[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) c16[m] = cmul(rc[ks][m], rstep[0][hh][ks][m]);
        rotate_pairs(cur.k[1][ks], cur.k[1][ks + NKS / 2], c16);
      }
      if (it + 1 < iters) {
        if ((it & 15) == 15) {
          load_angles(it + 1);
        } else {
#pragma unroll
          for (int ks = 0; ks < NKS / 2; ++ks)
#pragma unroll
            for (int m = 0; m < 4; ++m) rc[ks][m] = cmul(rc[ks][m], rstep[1][hh][ks][m]);
        }
      }
    }
    // ---- scores S^T: lane l holds head l%16, keys 16*gq + 4*(l/16) + r
    f32x4 s[2];
#pragma unroll
    for (int gq = 0; gq < 2; ++gq) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        acc = mfma16x16x32(__builtin_bit_cast(bf16x8, cur.k[gq][ks]), qf[ks], acc);
      s[gq] = acc;
    }
    // ---- start the next slice's loads while this one is finished
    if (it + 1 < iters) load_slice(ub + ((it + 1) * NW + wave) * kSlice, cur);

    float mx = -INFINITY;
#pragma unroll
    for (int gq = 0; gq < 2; ++gq)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = u0 + 16 * gq + 4 * hh + r;
        if (u >= ue) s[gq][r] = -INFINITY;
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
    // The V^T slice is this wave's own LDS region: its writes above complete
    // before the reads below (a wave's LDS operations run in order; the wait
    // also keeps the compiler from moving memory operations across), and the
    // next slice's writes come after these reads were consumed. No other wave
    // touches it until the merge, which starts with a barrier.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint16_t* vrow = vt + (16 * db + lane % 16) * VSTR + 8 * hh;
      const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vrow));
      oacc[db] = oacc[db] * corr;
      oacc[db] = mfma16x16x32(av, pb, oacc[db]);
    }
    asm volatile("" ::: "memory");
  }

  // ---- merge the waves: lane l holds head l%16, d = 16*db + 4*(l/16) + r;
  //      l_run is a partial sum over this lane group's keys.
  float lw = l_run;
  lw += __shfl_xor(lw, 16, kWave);
  lw += __shfl_xor(lw, 32, kWave);
  if (A.part != nullptr) {                      // split: this wave's partial, unnormalised
    if (lane % 16 < G) {
      float* pp = A.part + ((bg * A.np + split * NW + wave) * G + lane % 16) * part_stride<D>();
#pragma unroll
      for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4*>(pp + 4 + 16 * db + 4 * hh) = oacc[db];
      if (hh == 0) *reinterpret_cast<f32x2*>(pp) = f32x2{m_run, lw};
    }
    return;
  }
  __syncthreads();                              // every wave is done with its V^T slice
  float* red_o = reinterpret_cast<float*>(arena);   // [NW][16][D + 1], reuses the V^T slices
  if (lane < 16) {
    red_m[wave][lane] = m_run;
    red_l[wave][lane] = lw;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      red_o[(wave * 16 + lane % 16) * (D + 1) + 16 * db + 4 * hh + r] = oacc[db][r];
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    const int hq = e / D;
    const int d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, red_m[wv][hq]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      const float f = (red_m[wv][hq] == -INFINITY) ? 0.f : fast_exp2(red_m[wv][hq] - M);
      o += f * red_o[(wv * 16 + hq) * (D + 1) + d];
      l += f * red_l[wv][hq];
    }
    const int64_t orow = static_cast<int64_t>(b) * A.Hq + g * G + hq;
    const uint32_t bits = pack_bf16x2(o / l, 0.f);
    A.out[orow * D + d] = static_cast<uint16_t>(bits & 0xffffu);
    if (d == 0 && A.lse != nullptr) A.lse[orow] = (M + fast_log2(l)) * kLn2;
  }
}

// Merge of the np partials of kv head g of sequence b into out / lse: with
// M the largest partial max, o = sum_i 2^(m_i - M) o_i and l = sum_i
// 2^(m_i - M) l_i, out = o / l and lse = (M + log2 l) ln 2; a wave that saw
// no entry has m_i = -inf and weighs nothing. The partials are read kMB at a
// time, all loads issued before any is used, and blocks after the first are
// folded in with an online rescale.
template <int D>
__device__ __forceinline__ void merge_body(const DecodeArgs& A, int g, int b, int nthreads) {
  constexpr int PS = part_stride<D>();
  constexpr int kMB = 16;
  const int G = A.G;
  const int64_t bg = static_cast<int64_t>(b) * A.Hkv + g;
  for (int e = threadIdx.x; e < G * D; e += nthreads) {
    const int hq = e / D;
    const int d = e % D;
    const float* pp = A.part + bg * A.np * G * PS + hq * PS;
    float M = -INFINITY, o = 0.f, l = 0.f;
    for (int i0 = 0; i0 < A.np; i0 += kMB) {
      float mv[kMB], lv[kMB], ov[kMB];
#pragma unroll
      for (int k = 0; k < kMB; ++k) {
        const bool ok = i0 + k < A.np;
        const float* q = pp + static_cast<int64_t>(ok ? i0 + k : 0) * G * PS;
        const f32x2 ml = *reinterpret_cast<const f32x2*>(q);
        mv[k] = ok ? ml[0] : -INFINITY;
        lv[k] = ml[1];
        ov[k] = q[4 + d];
      }
      float Mb = M;
#pragma unroll
      for (int k = 0; k < kMB; ++k) Mb = fmaxf(Mb, mv[k]);
      if (M != -INFINITY && Mb != M) {
        const float f = fast_exp2(M - Mb);
        o *= f;
        l *= f;
      }
#pragma unroll
      for (int k = 0; k < kMB; ++k) {
        const float f = (mv[k] == -INFINITY) ? 0.f : fast_exp2(mv[k] - Mb);
        o += f * ov[k];
        l += f * lv[k];
      }
      M = Mb;
    }
    const int64_t orow = static_cast<int64_t>(b) * A.Hq + g * G + hq;
    const uint32_t bits = pack_bf16x2(o / l, 0.f);
    A.out[orow * D + d] = static_cast<uint16_t>(bits & 0xffffu);
    if (d == 0 && A.lse != nullptr) A.lse[orow] = (M + fast_log2(l)) * kLn2;
  }
}

// a split-decode workgroup: one 32-entry slice per wave and range unit
static_assert(kSplitWaves * kSlice == kSplitChunk, "split ranges are whole slices");

// the ranges of a split decode (decode.hip); their merge is a second launch
hipError_t launch_split_ranges(const DecodeArgs& A, const sep_cache& c, hipStream_t st);

inline DecodeArgs decode_args(const void* q, const void* k_new, const void* v_new, const sep_cache& c, int Hq,
                              float scale, const float* rope, void* out, float* lse) {
  DecodeArgs A;
  A.q = static_cast<const uint16_t*>(q);
  A.k_new = static_cast<const uint16_t*>(k_new);
  A.v_new = static_cast<const uint16_t*>(v_new);
  A.kc = static_cast<const uint16_t*>(c.k);
  A.vc = static_cast<const uint16_t*>(c.v);
  A.state = c.state;
  A.out = static_cast<uint16_t*>(out);
  A.lse = lse;
  A.rope = rope;
  A.part = nullptr;
  A.ns = 1;
  A.span = 0;
  A.np = 0;
  if (decode_uses_split(c, Hq)) {
    A.part = static_cast<float*>(c.work);
    decode_split_shape(c, &A.ns, &A.span);
    A.np = A.ns * kSplitWaves;
  }
  A.a = c.a;
  A.s = c.s;  // the separator-ring branch is only reached when cnt > 0, i.e. s >= 1
  A.p = c.p;
  A.w = c.w;
  A.rw = cache_ring(c);
  A.c = cache_slots(c);
  A.Hq = Hq;
  A.Hkv = c.Hkv;
  A.G = Hq / c.Hkv;
  A.scale_log2 = scale * kLog2e;
  return A;
}

}  // namespace sep
