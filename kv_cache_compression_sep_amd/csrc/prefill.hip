// sep_attn_prefill: fused Sep-Attention prefill for gfx950.
//
// What is computed (SepLLM pages: P2 §1.2, P1 "SepAttention"): for query
// head h of sequence b and key/value head g = h / (Hq/Hkv),
//   O[i] = sum_j softmax_j(scale * q_i . k_j over visible j) * v_j,
// where key j is visible to query i iff j <= i and (j < a, or i - j < n, or
// token j is a separator).
//
// How (P1 "Flex Attention Kernel": the speed-up only appears when the kernel
// itself sees the sparsity). A workgroup owns one query tile [q0, q1) of
// HPW heads that share a key/value head. With band_lo = max(q0 - n + 1, 0),
// every key j < band_lo is visible to all of the tile's queries iff it is
// initial or a separator, and invisible otherwise. So the tile reads:
//   * "global" keys: [0, min(a, band_lo)) followed by the separators in
//     [a, band_lo), gathered through the compacted list sep_pos
//     (rank[a] .. rank[band_lo]); no mask is needed on them;
//   * "band" keys [band_lo, q1) densely, with the element mask where a tile
//     is not fully visible.
// No other key is touched, so every fully masked block is skipped.
//
// Each wave holds NQB blocks of 32 query rows of one head. Scores are
// computed transposed, S^T = K Q^T, with the 32x32 MFMA so that each lane
// owns one query column: the row max is a max over the lane's values plus
// one exchange with lane l^32, and the exponentiated scores already sit in
// the B-operand layout of the P.V product (O^T = V^T P^T). Every K or V
// fragment read from LDS feeds the NQB blocks. K tiles are staged row-major
// in LDS; V tiles are staged transposed (d-major) with the key quads
// permuted so that each lane reads its eight keys with one 16-byte LDS read.
// Tiles are double buffered: the global loads of tile t+1 are in flight
// while tile t is computed, and the gather indices run two tiles ahead.
// Softmax is online in fp32 with exp2 (scale * log2 e folded in) and lazy
// rescaling: the running max only moves when some row's max grows by more
// than 8 (log2 units), so exponentials stay below 2^8.
#include "common.hpp"
#include "internal.hpp"

namespace sep {

// Query blocks of 32 rows per wave in the bf16 path (a build-time tuning
// constant: more blocks reuse each LDS fragment more often but need more
// registers per wave).
#ifndef SEPATTN_PREFILL_NQB
#define SEPATTN_PREFILL_NQB 1
#endif

constexpr int KT = 64;          // keys per tile
constexpr int NWAVES = 4;
constexpr int NTHREADS = NWAVES * kWave;
constexpr float kLazy = 8.0f;   // lazy-rescale threshold (log2 units)

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const uint8_t* is_sep;
  const int32_t* rank;
  const int32_t* sep_pos;
  int B, Hq, Hkv, S, a, n;
  int G, HPW, QT, n_hg, n_qt;
  float scale_log2;
};

// ---------------------------------------------------------------- traits
// bf16 inputs, 32x32x16 bf16 MFMA, NQB 32-row query blocks per wave.
template <int D_>
struct TraitsBF16 {
  static constexpr int D = D_;
  static constexpr int NQB = SEPATTN_PREFILL_NQB;
  static constexpr int KS = D / 16;             // k-steps of QK^T
  static constexpr int DB = D / 32;             // d-blocks of O^T
  static constexpr int KSTR = D + 8;            // K row stride (bf16)
  static constexpr int VSTR = KT + 8;           // V^T row stride (bf16)
  static constexpr int KBUF = KT * KSTR * 2;    // bytes
  static constexpr int VBUF = D * VSTR * 2;
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int KLOADS = KT * CPR / NTHREADS;
  static constexpr int MIN_WAVES = NQB == 1 ? 2 : 1;   // waves per SIMD the registers allow
  using elem = uint16_t;
  using qfrag = bf16x8;

  struct Stage {
    u32x4 kr[KLOADS];
    u32x4 vr[4];
  };

  __device__ static void load_q(const elem* qbase, int row, int lane, qfrag (&qf)[KS]) {
    const elem* p = qbase + static_cast<int64_t>(row) * D + 8 * (lane / 32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p + 16 * ks));
  }

  __device__ static void issue(const elem* kb, const elem* vb, const int32_t* idx, int tid,
                               Stage& st) {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int row = tid / CPR + i * (NTHREADS / CPR);
      const int c = tid % CPR;
      st.kr[i] = *reinterpret_cast<const u32x4*>(kb + static_cast<int64_t>(idx[row]) * D + 8 * c);
    }
    const int kq = tid % 16;
    const int dc = tid / 16;
    if (dc < CPR) {
      const int4 keys = *reinterpret_cast<const int4*>(idx + 4 * kq);
      st.vr[0] = *reinterpret_cast<const u32x4*>(vb + static_cast<int64_t>(keys.x) * D + 8 * dc);
      st.vr[1] = *reinterpret_cast<const u32x4*>(vb + static_cast<int64_t>(keys.y) * D + 8 * dc);
      st.vr[2] = *reinterpret_cast<const u32x4*>(vb + static_cast<int64_t>(keys.z) * D + 8 * dc);
      st.vr[3] = *reinterpret_cast<const u32x4*>(vb + static_cast<int64_t>(keys.w) * D + 8 * dc);
    }
  }

  __device__ static void store(char* kbuf, char* vbuf, int tid, const Stage& st) {
    elem* K = reinterpret_cast<elem*>(kbuf);
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int row = tid / CPR + i * (NTHREADS / CPR);
      const int c = tid % CPR;
      *reinterpret_cast<u32x4*>(K + row * KSTR + 8 * c) = st.kr[i];
    }
    const int kq = tid % 16;
    const int dc = tid / 16;
    if (dc < CPR) {
      // key quad kq -> column base, with quads 1 and 2 of each 16-key block
      // swapped (the order in which a lane's B operand holds its keys)
      const int qd = kq & 3;
      const int pq = (qd == 1) ? 2 : ((qd == 2) ? 1 : qd);
      const int col = 16 * (kq >> 2) + 4 * pq;
      elem* V = reinterpret_cast<elem*>(vbuf);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t w01e = __builtin_amdgcn_perm(st.vr[1][m], st.vr[0][m], 0x05040100u);
        const uint32_t w23e = __builtin_amdgcn_perm(st.vr[3][m], st.vr[2][m], 0x05040100u);
        const uint32_t w01o = __builtin_amdgcn_perm(st.vr[1][m], st.vr[0][m], 0x07060302u);
        const uint32_t w23o = __builtin_amdgcn_perm(st.vr[3][m], st.vr[2][m], 0x07060302u);
        const int d = 8 * dc + 2 * m;
        *reinterpret_cast<u32x2*>(V + d * VSTR + col) = u32x2{w01e, w23e};
        *reinterpret_cast<u32x2*>(V + (d + 1) * VSTR + col) = u32x2{w01o, w23o};
      }
    }
  }

  // S^T[qb] = K[keys 32*mb .. 32*mb+31] . Q^T[qb]
  __device__ static void qk_half(const char* kbuf, int lane, const qfrag (&qf)[NQB][KS], int mb,
                                 f32x16 (&s)[NQB]) {
    const elem* K = reinterpret_cast<const elem*>(kbuf);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) s[qb] = f32x16{};
    const elem* row = K + (32 * mb + lane % 32) * KSTR + 8 * (lane / 32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16 * ks));
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) s[qb] = mfma32x32x16(a, qf[qb][ks], s[qb]);
    }
  }

  // O^T[qb] += V^T[:, keys of half mb] . P^T[qb]; p holds the exponentiated
  // scores (fp32) of that half, rounded to bf16 here.
  __device__ static void pv_half(const char* vbuf, int lane, const f32x16 (&p)[NQB], int mb,
                                 f32x16 (&o)[NQB][DB]) {
    const elem* V = reinterpret_cast<const elem*>(vbuf);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int kc = 2 * mb + c2;
      bf16x8 b[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int r0 = 8 * c2;
        u32x4 pk;
        pk[0] = pack_bf16x2(p[qb][r0 + 0], p[qb][r0 + 1]);
        pk[1] = pack_bf16x2(p[qb][r0 + 2], p[qb][r0 + 3]);
        pk[2] = pack_bf16x2(p[qb][r0 + 4], p[qb][r0 + 5]);
        pk[3] = pack_bf16x2(p[qb][r0 + 6], p[qb][r0 + 7]);
        b[qb] = __builtin_bit_cast(bf16x8, pk);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const elem* vrow = V + (32 * db + lane % 32) * VSTR + 16 * kc + 8 * (lane / 32);
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vrow));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) o[qb][db] = mfma32x32x16(a, b[qb], o[qb][db]);
      }
    }
  }

  __device__ static void write_out(elem* dst, const float* vals4) {
    u32x2 w;
    w[0] = pack_bf16x2(vals4[0], vals4[1]);
    w[1] = pack_bf16x2(vals4[2], vals4[3]);
    *reinterpret_cast<u32x2*>(dst) = w;
  }
};

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
struct TileInfo {
  int band_lo, n_init, n_glob, rank_a, ntg, ntiles;
};

// Row to load for entry u of tile t (keys outside the list are clamped to a
// valid row; their scores are masked).
__device__ __forceinline__ int tile_key(const TileInfo& ti, const int32_t* sp, int S, int t, int u,
                                        bool* is_band) {
  if (t < ti.ntg) {
    *is_band = false;
    const int gu = t * KT + u;
    if (gu >= ti.n_glob) return 0;
    if (gu < ti.n_init) return gu;
    return sp[ti.rank_a + gu - ti.n_init];
  }
  *is_band = true;
  const int j = ti.band_lo + (t - ti.ntg) * KT + u;
  return j < S ? j : S - 1;
}

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

  // ---- work item: heavy (late) query tiles first; pairs that share K/V
  //      stay on one XCD (workgroups are dealt to the 8 XCDs round-robin).
  const int pairs = P.B * P.Hkv * P.n_hg;
  const int id = blockIdx.x;
  int pair, qt;
  if ((pairs % 8) == 0) {
    const int per = pairs / 8;
    const int xcd = id % 8;
    const int k = id / 8;
    pair = xcd + 8 * (k % per);
    qt = P.n_qt - 1 - k / per;
  } else {
    pair = id % pairs;
    qt = P.n_qt - 1 - id / pairs;
  }
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

  TileInfo ti;
  ti.band_lo = max(q0 - P.n + 1, 0);
  ti.n_init = min(P.a, ti.band_lo);
  ti.rank_a = rk[min(P.a, S)];
  const int n_sepg = (ti.band_lo > P.a) ? (rk[ti.band_lo] - ti.rank_a) : 0;
  ti.n_glob = ti.n_init + n_sepg;
  ti.ntg = (ti.n_glob + KT - 1) / KT;
  const int n_band = q1 - ti.band_lo;
  ti.ntiles = ti.ntg + (n_band + KT - 1) / KT;

  const elem* kb = reinterpret_cast<const elem*>(P.k) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const elem* vb = reinterpret_cast<const elem*>(P.v) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const elem* qb_ptr = reinterpret_cast<const elem*>(P.q) + static_cast<int64_t>(b * P.Hq + h) * S * D;

  // ---- index stage for tile t into slot t%3 (wave 0 only)
  auto index_load = [&](int t, int& key, uint64_t& bits) {
    bool band;
    key = tile_key(ti, sp, S, t, lane, &band);
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
        for (int qb = 0; qb < NQB; ++qb) {
          uint64_t m;
          if (band) {
            const int dq = qw0 + 32 * qb + lane % 32 - jmin;     // causal: u <= dq
            const int wl = dq - P.n + 1;                          // window: u >= wl
            const int ih = P.a - jmin;                            // initial: u < ih
            const uint64_t cm = dq >= 63 ? ~0ull : (dq < 0 ? 0ull : ((2ull << dq) - 1));
            const uint64_t wm = wl <= 0 ? ~0ull : (wl >= 64 ? 0ull : ~((1ull << wl) - 1));
            const uint64_t im = ih >= 64 ? ~0ull : (ih <= 0 ? 0ull : ((1ull << ih) - 1));
            m = cm & (wm | im | sepbits[t % 3]);
          } else {
            m = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1);
          }
          vis[qb] = m >> (4 * hsel);
        }
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
  A.a = a;
  A.n = n;
  A.G = Hq / Hkv;
  A.HPW = (A.G % 4 == 0) ? 4 : ((A.G % 2 == 0) ? 2 : 1);
  A.n_hg = A.G / A.HPW;
  A.scale_log2 = scale * kLog2e;
  if (dtype == SEP_BF16)
    return D == 128 ? launch<TraitsBF16<128>>(A, st) : launch<TraitsBF16<64>>(A, st);
  return D == 128 ? launch<TraitsF32<128>>(A, st) : launch<TraitsF32<64>>(A, st);
}

}  // namespace sep
