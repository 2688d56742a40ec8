// sep_attn_prefill: dispatch, and the fp32 path.
//
// What is computed (SepLLM pages: P2 §1.2, P1 "SepAttention"): for query
// head h of sequence b and key/value head g = h / (Hq/Hkv),
//   O[i] = sum_j softmax_j(scale * q_i . k_j over visible j) * v_j,
// where key j is visible to query i iff j <= i and (j < a, or i - j < n, or
// token j is a separator). The key list of a query tile (gathered initial
// and separator keys, then the dense band; prefill.hpp) is the same for
// both paths; bf16 runs in prefill_bf16.hip.
//
// fp32 path: full fp32 products on the 32x32x2 fp32 MFMA. A workgroup of
// four waves owns one query tile; each wave holds 32 query rows of one head.
// K tiles are staged in LDS with an odd row stride (conflict-free column
// reads); V tiles row-major (the fp32 PV operand needs one element per lane
// and key pair, so no transpose). Tiles are double buffered through
// registers; gather indices run two tiles ahead. Online softmax in fp32
// (exp2, lazy rescaling by more than 8 in log2 units).
#include "prefill.hpp"
#include "internal.hpp"

namespace sep {

constexpr int KT = 64;          // keys per tile
constexpr int NWAVES = 4;
constexpr int NTHREADS = NWAVES * kWave;
constexpr float kLazy = 8.0f;   // lazy-rescale threshold (log2 units)


// ---------------------------------------------------------------- traits
// fp32 inputs, 32x32x2 fp32 MFMA (full fp32 products), one query block.
template <int D_>
struct TraitsF32 {
  static constexpr int D = D_;
  static constexpr int NQB = 1;
  static constexpr int KS = D / 2;
  static constexpr int DB = D / 32;
  static constexpr int KSTR = D + 1;            // odd stride: conflict-free column reads
  static constexpr int VSTR = D;
  static constexpr int KBUF = KT * KSTR * 4;
  static constexpr int VBUF = KT * VSTR * 4;
  static constexpr int CPR = D / 4;             // 16-byte chunks per row
  static constexpr int LOADS = KT * CPR / NTHREADS;
  static constexpr int MIN_WAVES = 1;
  using elem = float;
  using qfrag = float;

  struct Stage {
    f32x4 kr[LOADS];
    f32x4 vr[LOADS];
  };

  __device__ static void load_q(const elem* qbase, int row, int lane, qfrag (&qf)[KS]) {
    const elem* p = qbase + static_cast<int64_t>(row) * D + (lane / 32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = p[2 * ks];
  }

  __device__ static void issue(const elem* kb, const elem* vb, const int32_t* idx, int tid,
                               Stage& st) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = tid / CPR + i * (NTHREADS / CPR);
      const int c = tid % CPR;
      const int64_t off = static_cast<int64_t>(idx[row]) * D + 4 * c;
      st.kr[i] = *reinterpret_cast<const f32x4*>(kb + off);
      st.vr[i] = *reinterpret_cast<const f32x4*>(vb + off);
    }
  }

  __device__ static void store(char* kbuf, char* vbuf, int tid, const Stage& st) {
    float* K = reinterpret_cast<float*>(kbuf);
    float* V = reinterpret_cast<float*>(vbuf);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = tid / CPR + i * (NTHREADS / CPR);
      const int c = tid % CPR;
#pragma unroll
      for (int e = 0; e < 4; ++e) K[row * KSTR + 4 * c + e] = st.kr[i][e];
      *reinterpret_cast<f32x4*>(V + row * VSTR + 4 * c) = st.vr[i];
    }
  }

  __device__ static void qk_half(const char* kbuf, int lane, const qfrag (&qf)[NQB][KS], int mb,
                                 f32x16 (&s)[NQB]) {
    const float* K = reinterpret_cast<const float*>(kbuf);
    f32x16 acc = {};
    const float* row = K + (32 * mb + lane % 32) * KSTR + (lane / 32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mfma32x32x2f32(row[2 * ks], qf[0][ks], acc);
    s[0] = acc;
  }

  __device__ static void pv_half(const char* vbuf, int lane, const f32x16 (&p)[NQB], int mb,
                                 f32x16 (&o)[NQB][DB]) {
    const float* V = reinterpret_cast<const float*>(vbuf);
    const int h = lane / 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * mb + 8 * (r / 4) + 4 * h + (r % 4);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[0][db] = mfma32x32x2f32(V[key * VSTR + 32 * db + lane % 32], p[0][r], o[0][db]);
    }
  }

  __device__ static void write_out(elem* dst, const float* vals4) {
    *reinterpret_cast<f32x4*>(dst) = f32x4{vals4[0], vals4[1], vals4[2], vals4[3]};
  }
};

// ---------------------------------------------------------------- driver
template <class Tr>
__global__ void __launch_bounds__(NTHREADS, Tr::MIN_WAVES) prefill_kernel(PrefillArgs P) {
  using elem = typename Tr::elem;
  constexpr int D = Tr::D;
  constexpr int DB = Tr::DB;
  constexpr int NQB = Tr::NQB;
  constexpr int QW = 32 * NQB;                  // query rows per wave

  // One LDS arena: double-buffered K and V tiles during the key loop, the
  // normalised output tile (one 32-row block per wave at a time) at the end.
  constexpr int OSTR = D + 4;                   // fp32 output-staging row stride
  constexpr int ARENA = 2 * Tr::KBUF + 2 * Tr::VBUF;
  static_assert(NWAVES * 32 * OSTR * 4 <= ARENA, "output staging must fit the arena");
  __shared__ __attribute__((aligned(16))) char arena[ARENA];
  __shared__ __attribute__((aligned(16))) int32_t idxbuf[3][KT];
  __shared__ uint64_t sepbits[3];
  auto kbuf = [&](int i) -> char* { return arena + i * Tr::KBUF; };
  auto vbuf = [&](int i) -> char* { return arena + 2 * Tr::KBUF + i * Tr::VBUF; };

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;

  int pair, qt;
  work_item(P, blockIdx.x, &pair, &qt);
  const int hg = pair % P.n_hg;
  const int bg = pair / P.n_hg;
  const int g = bg % P.Hkv;
  const int b = bg / P.Hkv;
  const int S = P.S;
  const int q0 = qt * P.QT;
  const int q1 = min(q0 + P.QT, S);

  const int hw = wave % P.HPW;
  const int rb = wave / P.HPW;
  const int h = g * P.G + hg * P.HPW + hw;
  const int qw0 = q0 + QW * rb;                 // first query row of this wave

  const int32_t* rk = P.rank + static_cast<int64_t>(b) * (S + 1);
  const int32_t* sp = P.sep_pos + static_cast<int64_t>(b) * S;
  const uint8_t* fl = P.is_sep + static_cast<int64_t>(b) * S;

  const TileInfo ti = tile_info<KT>(rk, S, P.a, P.n, q0, q1);

  const elem* kb = reinterpret_cast<const elem*>(P.k) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const elem* vb = reinterpret_cast<const elem*>(P.v) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const elem* qb_ptr = reinterpret_cast<const elem*>(P.q) + static_cast<int64_t>(b * P.Hq + h) * S * D;

  // ---- index stage for tile t into slot t%3 (wave 0 only)
  auto index_load = [&](int t, int& key, uint64_t& bits) {
    bool band;
    key = tile_key<KT>(ti, sp, S, t, lane, &band);
    bool f = false;
    if (band) {
      const int j = ti.band_lo + (t - ti.ntg) * KT + lane;
      f = (j < S) && (fl[j] != 0);
    }
    bits = ballot(f);
  };
  auto index_store = [&](int t, int key, uint64_t bits) {
    idxbuf[t % 3][lane] = key;
    if (lane == 0) sepbits[t % 3] = bits;
  };

  if (wave == 0) {
    int key;
    uint64_t bits;
    index_load(0, key, bits);
    index_store(0, key, bits);
    if (ti.ntiles > 1) {
      index_load(1, key, bits);
      index_store(1, key, bits);
    }
  }
  __syncthreads();
  typename Tr::Stage st;
  Tr::issue(kb, vb, idxbuf[0], tid, st);
  Tr::store(kbuf(0), vbuf(0), tid, st);

  // ---- per-wave query state
  typename Tr::qfrag qf[NQB][Tr::KS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
    Tr::load_q(qb_ptr, min(qw0 + 32 * qb + lane % 32, S - 1), lane, qf[qb]);
  f32x16 oacc[NQB][DB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16{};
  float m_run[NQB], l_run[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
  }
  const int qmax = min(qw0 + QW - 1, S - 1);
  const int hsel = lane / 32;

  for (int t = 0; t < ti.ntiles; ++t) {
    __syncthreads();
    const int cur = t & 1;
    if (t + 1 < ti.ntiles) Tr::issue(kb, vb, idxbuf[(t + 1) % 3], tid, st);
    int nkey = 0;
    uint64_t nbits = 0;
    const bool more_idx = (wave == 0) && (t + 2 < ti.ntiles);
    if (more_idx) index_load(t + 2, nkey, nbits);

    // ---- classify this tile for this wave
    const bool band = t >= ti.ntg;
    const int jmin = band ? ti.band_lo + (t - ti.ntg) * KT : 0;
    const int nvalid = band ? KT : min(KT, ti.n_glob - t * KT);
    bool skip = false, need_mask = false;
    if (band) {
      if (jmin > qmax || qw0 >= S) skip = true;            // every key in the future
      else need_mask = !(jmin + KT - 1 <= qw0 && jmin >= qmax - P.n + 1);
    } else {
      need_mask = nvalid < KT;
    }

    if (!skip) {
      // Visibility of this lane's keys, one bit per key of the tile, shifted
      // so that bit u0 stands for key u0 + 4*hsel (the lane's key for
      // register r of half mb is u0 = 32*mb + 8*(r/4) + r%4).
      uint64_t vis[NQB];
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          vis[qb] = vis_word(band, qw0 + 32 * qb + lane % 32, jmin, P.n, P.a, sepbits[t % 3],
                             nvalid) >> (4 * hsel);
      }
      f32x16 sh[2][NQB];
      Tr::qk_half(kbuf(cur), lane, qf, 0, sh[0]);
      Tr::qk_half(kbuf(cur), lane, qf, 1, sh[1]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 (&s)[NQB] = sh[mb];
        if (need_mask) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            const uint32_t word = static_cast<uint32_t>(vis[qb] >> (32 * mb));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const uint32_t bit = 1u << (8 * (r / 4) + (r % 4));
              s[qb][r] = (word & bit) ? s[qb][r] : -INFINITY;
            }
          }
        }
        // ---- online softmax over this half (log2 domain), lazily rescaled
        float mx[NQB];
        bool grow = false;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          float m = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, s[qb][r]);
          mx[qb] = fmaxf(m, swap_half(m)) * P.scale_log2;
          grow |= mx[qb] > m_run[qb] + kLazy;
        }
        if (ballot(grow) != 0ull) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            const float m_new = fmaxf(m_run[qb], mx[qb]);
            const float corr = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run[qb] - m_new);
            l_run[qb] *= corr;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[qb][db] *= corr;
            m_run[qb] = m_new;
          }
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const float msub = (m_run[qb] == -INFINITY) ? 0.0f : m_run[qb];
          float lsum = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = fast_exp2(__builtin_fmaf(s[qb][r], P.scale_log2, -msub));
            s[qb][r] = pv;
            lsum += pv;
          }
          l_run[qb] += lsum;
        }
        Tr::pv_half(vbuf(cur), lane, s, mb, oacc);
      }
    }

    if (t + 1 < ti.ntiles) Tr::store(kbuf(cur ^ 1), vbuf(cur ^ 1), tid, st);
    if (more_idx) index_store(t + 2, nkey, nbits);
  }

  // ---- epilogue: normalise, stage one 32-row block per wave through LDS,
  //      store coalesced rows
  elem* ob = reinterpret_cast<elem*>(P.out) + static_cast<int64_t>(b * P.Hq + h) * S * D;
  float* slice = reinterpret_cast<float*>(arena) + wave * (32 * OSTR);
  constexpr int C4 = D / 4;                     // 4-element groups per row
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float l_tot = l_run[qb] + swap_half(l_run[qb]);
    const float inv = 1.0f / l_tot;
    __syncthreads();
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * db + 8 * j + 4 * hsel;
        *reinterpret_cast<f32x4*>(slice + (lane % 32) * OSTR + d0) =
            f32x4{oacc[qb][db][4 * j] * inv, oacc[qb][db][4 * j + 1] * inv,
                  oacc[qb][db][4 * j + 2] * inv, oacc[qb][db][4 * j + 3] * inv};
      }
    __syncthreads();
    const int r0 = qw0 + 32 * qb;
    for (int e = lane; e < 32 * C4; e += kWave) {
      const int r = e / C4;
      const int c = e % C4;
      const int row = r0 + r;
      if (row < S) Tr::write_out(ob + static_cast<int64_t>(row) * D + 4 * c, slice + r * OSTR + 4 * c);
    }
    const int qi = r0 + lane % 32;
    if (P.lse != nullptr && lane < 32 && qi < S)
      P.lse[static_cast<int64_t>(b * P.Hq + h) * S + qi] = (m_run[qb] + fast_log2(l_tot)) * kLn2;
  }
}

template <class Tr>
static hipError_t launch(PrefillArgs A, hipStream_t st) {
  A.QT = 32 * Tr::NQB * (NWAVES / A.HPW);
  A.n_qt = (A.S + A.QT - 1) / A.QT;
  const int grid = A.B * A.Hkv * A.n_hg * A.n_qt;
  hipLaunchKernelGGL(prefill_kernel<Tr>, dim3(grid), dim3(NTHREADS), 0, st, A);
  return hipGetLastError();
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                          int Hkv, int S, int D, const uint8_t* is_sep, const int32_t* rank,
                          const int32_t* sep_pos, int a, int n, float scale, void* out, float* lse,
                          hipStream_t st) {
  PrefillArgs A;
  A.q = q;
  A.k = k;
  A.v = v;
  A.out = out;
  A.lse = lse;
  A.is_sep = is_sep;
  A.rank = rank;
  A.sep_pos = sep_pos;
  A.B = B;
  A.Hq = Hq;
  A.Hkv = Hkv;
  A.S = S;
  A.Skv = S;
  A.q_base = 0;
  A.key_lo = nullptr;
  A.a = a;
  A.n = n;
  A.G = Hq / Hkv;
  A.HPW = (A.G % 4 == 0) ? 4 : ((A.G % 2 == 0) ? 2 : 1);
  A.n_hg = A.G / A.HPW;
  A.scale_log2 = scale * kLog2e;
  if (dtype == SEP_BF16) return launch_prefill_bf16(A, D, st);
  return D == 128 ? launch<TraitsF32<128>>(A, st) : launch<TraitsF32<64>>(A, st);
}

}  // namespace sep
