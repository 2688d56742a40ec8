// sep_attn_prefill_backward: gradients of Sep-Attention prefill.
//
// For L = sum(dO * O) (SepLLM pages: P2 §1.2 scaled masked softmax attention;
// P1 "Training-SepLLM" trains through the same mask), with P the softmax
// weights of query head h over kv head g = h / G:
//   delta_i = sum_d dO_id O_id
//   dP = dO V^T,  dS = P * (dP - delta),  dQ = scale dS K,
//   dV_g = sum_h P^T dO,  dK_g = scale sum_h dS^T Q.
// P is recomputed from the forward's lse: P_ij = exp(scale q_i.k_j - lse_i)
// on visible pairs (j <= i and (j < a, or i - j < n, or j a separator)).
//
// Everything is fp32 (inputs bf16 or fp32, widened exactly), on the
// 32x32x2 fp32 MFMA:
//   delta_kernel  one 16-lane group per query row.
//   dq_kernel     the forward's decomposition: a workgroup owns 32 query
//                 rows of each of 4 heads and walks their key list (the
//                 gathered initial + separator keys, then the band) in tiles
//                 of 64; S^T = K Q^T and dP^T = V dO^T as in the forward, then
//                 dQ^T += K^T dS^T.
//   dkdv_band     one workgroup per 128 consecutive keys (32 per wave) of a
//                 kv head: it walks the queries of their windows, [j0, j0 +
//                 127 + n), for every head of the group; initial and
//                 separator keys are masked out here. S = Q K^T puts one key
//                 per lane, so dV^T += dO^T P and dK^T += Q^T dS take the
//                 query rows from LDS. Plain stores: every row of dK and dV.
//   dkdv_glob     the initial and separator keys, which every later query
//                 sees: a work item is (kv head, 256-query chunk, tile of 128
//                 gathered keys that start before the chunk's end); it adds
//                 its partial dK / dV with fp32 atomics, after dkdv_band.
#include "prefill_bwd.hpp"

#include <type_traits>

namespace sep {
namespace {
using namespace bwd;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

template <class T>
struct Ld;
template <>
struct Ld<float> {
  __device__ static f32x4 four(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
};
template <>
struct Ld<uint16_t> {
  __device__ static f32x4 four(const uint16_t* p) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    return f32x4{bf16lo(w[0]), bf16hi(w[0]), bf16lo(w[1]), bf16hi(w[1])};
  }
};

// ---------------------------------------------------------------- delta
template <class T, int D>
__global__ void __launch_bounds__(256) delta_kernel(BwdArgs P) {
  const int64_t rows = static_cast<int64_t>(P.B) * P.Hq * P.S;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 16 + threadIdx.x / 16;
  const int sub = threadIdx.x % 16;
  float acc = 0.f;
  if (row < rows) {
    const T* o = reinterpret_cast<const T*>(P.out) + row * D;
    const T* d = reinterpret_cast<const T*>(P.dout) + row * D;
#pragma unroll
    for (int c = sub * 4; c < D; c += 64) {
      const f32x4 x = Ld<T>::four(o + c), y = Ld<T>::four(d + c);
      acc += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < rows && sub == 0) P.delta[row] = acc;
}

// ---------------------------------------------------------------- dQ
template <class T, int D>
__global__ void __launch_bounds__(BT, 1) dq_kernel(BwdArgs P) {
  constexpr int KS = D / 2;
  constexpr int DB = D / 32;
  constexpr int STR = D + 1;                      // odd stride: conflict-free column reads
  constexpr int CPR = D / 4;
  constexpr int LOADS = KTQ * CPR / BT;
  __shared__ float Kt[KTQ * STR];
  __shared__ float Vt[KTQ * STR];
  __shared__ int32_t idxbuf[2][KTQ];
  __shared__ uint64_t sepbits[2];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int hsel = lane / 32;

  PrefillArgs W;                                  // the forward's work-item mapping
  W.B = P.B; W.Hkv = P.Hkv; W.n_hg = P.n_hg; W.n_qt = P.n_qt;
  int pair, qt;
  work_item(W, blockIdx.x, &pair, &qt);
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
  const int qw0 = q0 + 32 * rb;
  const int qmax = min(qw0 + 31, S - 1);

  const int32_t* rk = P.rank + static_cast<int64_t>(b) * (S + 1);
  const int32_t* sp = P.sep_pos + static_cast<int64_t>(b) * S;
  const uint8_t* fl = P.is_sep + static_cast<int64_t>(b) * S;
  const TileInfo ti = tile_info<KTQ>(rk, S, P.a, P.n, q0, q1);

  const T* kb = reinterpret_cast<const T*>(P.k) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const T* vb = reinterpret_cast<const T*>(P.v) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const int64_t hrow = static_cast<int64_t>(b * P.Hq + h) * S;

  // query column of this lane: Q^T and dO^T fragments, lse (log2), delta
  const int qi = qw0 + lane % 32;
  const int qc = min(qi, S - 1);
  float qf[KS], of[KS];
  {
    const T* qp = reinterpret_cast<const T*>(P.q) + (hrow + qc) * D;
    const T* op = reinterpret_cast<const T*>(P.dout) + (hrow + qc) * D;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      const f32x4 x = Ld<T>::four(qp + c), y = Ld<T>::four(op + c);
      // element d = 2 ks + hsel of this lane's row
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (((c + e) & 1) == hsel) {
          qf[(c + e) / 2] = x[e];
          of[(c + e) / 2] = y[e];
        }
      }
    }
  }
  const float lse2 = P.lse[hrow + qc] * kLog2e;
  const float dlt = P.delta[hrow + qc];

  auto index_load = [&](int t, int& key, uint64_t& bits) {
    bool band;
    key = tile_key<KTQ>(ti, sp, S, t, lane, &band);
    bool f = false;
    if (band) {
      const int j = ti.band_lo + (t - ti.ntg) * KTQ + lane;
      f = (j < S) && (fl[j] != 0);
    }
    bits = ballot(f);
  };
  if (wave == 0 && ti.ntiles > 0) {
    int key;
    uint64_t bits;
    index_load(0, key, bits);
    idxbuf[0][lane] = key;
    if (lane == 0) sepbits[0] = bits;
  }
  __syncthreads();

  f32x16 dacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dacc[db] = f32x16{};

  for (int t = 0; t < ti.ntiles; ++t) {
    // rows of tile t into registers; the index of tile t + 1 meanwhile
    f32x4 kr[LOADS], vr[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = tid / CPR + i * (BT / CPR);
      const int c = tid % CPR;
      const int64_t off = static_cast<int64_t>(idxbuf[t & 1][row]) * D + 4 * c;
      kr[i] = Ld<T>::four(kb + off);
      vr[i] = Ld<T>::four(vb + off);
    }
    int nkey = 0;
    uint64_t nbits = 0;
    const bool more = (wave == 0) && (t + 1 < ti.ntiles);
    if (more) index_load(t + 1, nkey, nbits);
    __syncthreads();                              // every wave is done with the previous tile
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = tid / CPR + i * (BT / CPR);
      const int c = tid % CPR;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Kt[row * STR + 4 * c + e] = kr[i][e];
        Vt[row * STR + 4 * c + e] = vr[i][e];
      }
    }
    if (more) {
      idxbuf[(t + 1) & 1][lane] = nkey;
      if (lane == 0) sepbits[(t + 1) & 1] = nbits;
    }
    __syncthreads();

    const bool band = t >= ti.ntg;
    const int jmin = band ? ti.band_lo + (t - ti.ntg) * KTQ : 0;
    const int nvalid = band ? KTQ : min(KTQ, ti.n_glob - t * KTQ);
    bool skip = false, need_mask = false;
    if (band) {
      if (jmin > qmax || qw0 >= S) skip = true;
      else need_mask = !(jmin + KTQ - 1 <= qw0 && jmin >= qmax - P.n + 1);
    } else {
      need_mask = nvalid < KTQ;
    }
    if (skip) continue;
    const uint64_t vis =
        need_mask ? (vis_word(band, qi, jmin, P.n, P.a, sepbits[t & 1], nvalid) >> (4 * hsel)) : ~0ull;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      // S^T and dP^T of keys 32 mb .. 32 mb + 31 (rows) x this wave's queries
      f32x16 s = {}, dp = {};
      const float* kr0 = Kt + (32 * mb + lane % 32) * STR + hsel;
      const float* vr0 = Vt + (32 * mb + lane % 32) * STR + hsel;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32x32x2f32(kr0[2 * ks], qf[ks], s);
        dp = mfma32x32x2f32(vr0[2 * ks], of[ks], dp);
      }
      const uint32_t word = static_cast<uint32_t>(vis >> (32 * mb));
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool on = (word >> (8 * (r / 4) + (r % 4))) & 1u;
        const float p = on ? fast_exp2(__builtin_fmaf(s[r], P.scale_log2, -lse2)) : 0.0f;
        ds[r] = p * (dp[r] - dlt);
      }
      // dQ^T += K^T dS^T over these 32 keys
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * mb + 8 * (r / 4) + 4 * hsel + (r % 4);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dacc[db] = mfma32x32x2f32(Kt[key * STR + 32 * db + lane % 32], ds[r], dacc[db]);
      }
    }
  }
  // lane: query column qi; rows d = 32 db + 8 (r / 4) + 4 hsel + r % 4
  if (qi < S) {
    float* dst = P.dq + (hrow + qi) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * j + 4 * hsel) =
            f32x4{dacc[db][4 * j] * P.scale, dacc[db][4 * j + 1] * P.scale, dacc[db][4 * j + 2] * P.scale,
                  dacc[db][4 * j + 3] * P.scale};
  }
}

// ---------------------------------------------------------------- dK, dV
// One query tile (32 rows of head h from row qt0) against this wave's 32
// keys: S = Q K^T (rows = queries, one key per lane), dP = dO V^T, then
// dV^T += dO^T P and dK^T += Q^T dS. Qt/Ot hold the tile's rows (rows past
// S are zero and masked); lse2/dlt the rows' log2 lse and delta.
template <int D, class Vis>
__device__ __forceinline__ void kv_tile(const float* Qt, const float* Ot, const float* lse2, const float* dlt,
                                        const float (&kf)[D / 2], const float (&vf)[D / 2], float scale_log2,
                                        int lane, Vis visible, f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32]) {
  constexpr int KS = D / 2;
  constexpr int DB = D / 32;
  constexpr int STR = D + 1;
  const int hsel = lane / 32;
  f32x16 s = {}, dp = {};
  const float* q0 = Qt + (lane % 32) * STR + hsel;
  const float* o0 = Ot + (lane % 32) * STR + hsel;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    s = mfma32x32x2f32(q0[2 * ks], kf[ks], s);
    dp = mfma32x32x2f32(o0[2 * ks], vf[ks], dp);
  }
  f32x16 p, ds;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int il = 8 * (r / 4) + 4 * hsel + (r % 4);   // query row of element r
    const float pv = visible(il) ? fast_exp2(__builtin_fmaf(s[r], scale_log2, -lse2[il])) : 0.0f;
    p[r] = pv;
    ds[r] = pv * (dp[r] - dlt[il]);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int il = 8 * (r / 4) + 4 * hsel + (r % 4);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dv[db] = mfma32x32x2f32(Ot[il * STR + 32 * db + lane % 32], p[r], dv[db]);
      dk[db] = mfma32x32x2f32(Qt[il * STR + 32 * db + lane % 32], ds[r], dk[db]);
    }
  }
}

// Stage query rows [qt0, qt0 + 32) of row block `hrow` (Q and dO, with lse
// and delta) into LDS; rows at or past S become zero.
template <class T, int D>
__device__ __forceinline__ void stage_queries(const BwdArgs& P, int64_t hrow, int qt0, float* Qt, float* Ot,
                                              float* lse2, float* dlt) {
  constexpr int STR = D + 1;
  constexpr int CPR = D / 4;
  const int tid = threadIdx.x;
  f32x4 xq[QB * CPR / BT], xo[QB * CPR / BT];
#pragma unroll
  for (int i = 0; i < QB * CPR / BT; ++i) {
    const int row = tid / CPR + i * (BT / CPR);
    const int c = tid % CPR;
    const int qr = qt0 + row;
    if (qr < P.S) {
      xq[i] = Ld<T>::four(reinterpret_cast<const T*>(P.q) + (hrow + qr) * D + 4 * c);
      xo[i] = Ld<T>::four(reinterpret_cast<const T*>(P.dout) + (hrow + qr) * D + 4 * c);
    } else {
      xq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      xo[i] = xq[i];
    }
  }
  float l = 0.f, d = 0.f;
  if (tid < QB && qt0 + tid < P.S) {
    l = P.lse[hrow + qt0 + tid] * kLog2e;
    d = P.delta[hrow + qt0 + tid];
  }
  __syncthreads();                                // the previous tile is consumed
#pragma unroll
  for (int i = 0; i < QB * CPR / BT; ++i) {
    const int row = tid / CPR + i * (BT / CPR);
    const int c = tid % CPR;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Qt[row * STR + 4 * c + e] = xq[i][e];
      Ot[row * STR + 4 * c + e] = xo[i][e];
    }
  }
  if (tid < QB) {
    lse2[tid] = l;
    dlt[tid] = d;
  }
  __syncthreads();
}

// K^T and V^T fragments of key j (this lane's key column): element d =
// 2 ks + hsel
template <class T, int D>
__device__ __forceinline__ void load_key(const T* kb, const T* vb, int j, int lane, float (&kf)[D / 2],
                                         float (&vf)[D / 2]) {
  const int hsel = lane / 32;
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    const f32x4 x = Ld<T>::four(kb + static_cast<int64_t>(j) * D + c);
    const f32x4 y = Ld<T>::four(vb + static_cast<int64_t>(j) * D + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (((c + e) & 1) == hsel) {
        kf[(c + e) / 2] = x[e];
        vf[(c + e) / 2] = y[e];
      }
    }
  }
}

template <class T, int D>
__global__ void __launch_bounds__(BT, 1) dkdv_band_kernel(BwdArgs P, int n_kt) {
  constexpr int KS = D / 2;
  constexpr int DB = D / 32;
  constexpr int STR = D + 1;
  __shared__ float Qt[QB * STR];
  __shared__ float Ot[QB * STR];
  __shared__ float lse2[QB], dlt[QB];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int hsel = lane / 32;
  const int kt = blockIdx.x % n_kt;
  const int bgi = blockIdx.x / n_kt;
  const int g = bgi % P.Hkv;
  const int b = bgi / P.Hkv;
  const int S = P.S;
  const int j0 = kt * KB;
  const int j = j0 + 32 * wave + lane % 32;      // this lane's key
  const int jc = min(j, S - 1);
  const uint8_t* fl = P.is_sep + static_cast<int64_t>(b) * S;
  // initial and separator keys are every later query's: dkdv_glob has them
  const bool own = j < S && j >= P.a && fl[jc] == 0;
  const T* kb = reinterpret_cast<const T*>(P.k) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const T* vb = reinterpret_cast<const T*>(P.v) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  float kf[KS], vf[KS];
  load_key<T, D>(kb, vb, jc, lane, kf, vf);
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  // queries of these keys' windows: [j0, j0 + KB - 1 + n), capped at S
  const int64_t qend64 = static_cast<int64_t>(j0) + KB - 1 + P.n;
  const int qend = static_cast<int>(qend64 < S ? qend64 : S);
  const int wj0 = j0 + 32 * wave;                 // this wave's first key
  for (int hh = 0; hh < P.G; ++hh) {
    const int64_t hrow = static_cast<int64_t>(b * P.Hq + g * P.G + hh) * S;
    for (int qt0 = j0; qt0 < qend; qt0 += QB) {
      stage_queries<T, D>(P, hrow, qt0, Qt, Ot, lse2, dlt);
      // this wave's keys see none of these rows: all rows before its first
      // key, or past the windows of all of them
      if (qt0 + QB - 1 < wj0 || static_cast<int64_t>(qt0) > static_cast<int64_t>(wj0) + 31 + P.n - 1) continue;
      kv_tile<D>(Qt, Ot, lse2, dlt, kf, vf, P.scale_log2, lane,
                 [&](int il) {
                   const int i = qt0 + il;
                   return own && i < S && i >= j && i - j < P.n;
                 },
                 dk, dv);
    }
  }
  if (j < S) {
    float* dkr = P.dk + (static_cast<int64_t>(b * P.Hkv + g) * S + j) * D;
    float* dvr = P.dv + (static_cast<int64_t>(b * P.Hkv + g) * S + j) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 32 * db + 8 * q + 4 * hsel;
        *reinterpret_cast<f32x4*>(dkr + d) = f32x4{dk[db][4 * q] * P.scale, dk[db][4 * q + 1] * P.scale,
                                                   dk[db][4 * q + 2] * P.scale, dk[db][4 * q + 3] * P.scale};
        *reinterpret_cast<f32x4*>(dvr + d) = f32x4{dv[db][4 * q], dv[db][4 * q + 1], dv[db][4 * q + 2],
                                                   dv[db][4 * q + 3]};
      }
  }
}

// Work items of dkdv_glob: (query chunk c, tile of KB global keys that start
// before the chunk's end). A workgroup first counts the tiles of every chunk
// of its sequence (from rank) into an exclusive prefix in LDS, then takes
// items w = slot, slot + nslots, ... and finds each item's chunk by binary
// search, so that the grid stays at the resident size whatever the separator
// density.
template <class T, int D>
__global__ void __launch_bounds__(BT, 1) dkdv_glob_kernel(BwdArgs P, int n_qc, int nslots) {
  constexpr int KS = D / 2;
  constexpr int DB = D / 32;
  constexpr int STR = D + 1;
  __shared__ float Qt[QB * STR];
  __shared__ float Ot[QB * STR];
  __shared__ float lse2[QB], dlt[QB];
  __shared__ int32_t kpos[KB];
  __shared__ int32_t tstart[kMaxChunks + 1];
  __shared__ int32_t wsum[BW];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int hsel = lane / 32;
  const int BH = P.B * P.Hkv;
  const int bgi = blockIdx.x % BH;                // a (sequence, kv head) per XCD where BH divides 8
  const int slot = blockIdx.x / BH;
  const int g = bgi % P.Hkv;
  const int b = bgi / P.Hkv;
  const int S = P.S;
  const int32_t* rk = P.rank + static_cast<int64_t>(b) * (S + 1);
  const int32_t* sp = P.sep_pos + static_cast<int64_t>(b) * S;
  const int ninit = min(P.a, S);
  const int rank_a = rk[ninit];
  // global keys before the end c1 of a chunk: initial [0, min(a, c1)), then
  // the separators in [a, c1)
  auto n_global = [&](int c1) { return min(ninit, c1) + (c1 > ninit ? rk[c1] - rank_a : 0); };

  const int total = chunk_tile_prefix(n_global, S, n_qc, tstart, wsum);

  const T* kb = reinterpret_cast<const T*>(P.k) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const T* vb = reinterpret_cast<const T*>(P.v) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  float* dkb = P.dk + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  float* dvb = P.dv + static_cast<int64_t>(b * P.Hkv + g) * S * D;

  for (int w = slot; w < total; w += nslots) {
    const int qc = chunk_of(tstart, n_qc, w);
    const int u0 = (w - tstart[qc]) * KB;
    const int c0 = qc * QCH;
    const int c1 = min(c0 + QCH, S);
    const int n_in = min(ninit, c1);
    const int n_gl = n_global(c1);
    __syncthreads();                              // kpos of the previous item is consumed
    for (int u = tid; u < KB; u += BT) {
      const int uu = u0 + u;
      kpos[u] = uu >= n_gl ? -1 : (uu < n_in ? uu : sp[rank_a + (uu - n_in)]);
    }
    __syncthreads();
    const int j = kpos[32 * wave + lane % 32];    // this lane's key, -1 past the list
    const int jc = j < 0 ? 0 : j;
    float kf[KS], vf[KS];
    load_key<T, D>(kb, vb, jc, lane, kf, vf);
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dk[db] = f32x16{};
      dv[db] = f32x16{};
    }
    const int jlo = kpos[0];                      // the tile's first (smallest) key
    const int wlo = kpos[32 * wave];              // this wave's first key (-1: none)
    const int qs = max(c0, jlo) / QB * QB;        // first query tile that can see a key
    for (int hh = 0; hh < P.G; ++hh) {
      const int64_t hrow = static_cast<int64_t>(b * P.Hq + g * P.G + hh) * S;
      for (int qt0 = qs; qt0 < c1; qt0 += QB) {
        stage_queries<T, D>(P, hrow, qt0, Qt, Ot, lse2, dlt);
        if (wlo < 0 || qt0 + QB - 1 < wlo) continue;
        kv_tile<D>(Qt, Ot, lse2, dlt, kf, vf, P.scale_log2, lane,
                   [&](int il) {
                     const int i = qt0 + il;
                     return j >= 0 && i >= c0 && i < c1 && i >= j;
                   },
                   dk, dv);
      }
    }
    if (j >= 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = 32 * db + 8 * (r / 4) + 4 * hsel + (r % 4);
          atomicAdd(dkb + static_cast<int64_t>(j) * D + d, dk[db][r] * P.scale);
          atomicAdd(dvb + static_cast<int64_t>(j) * D + d, dv[db][r]);
        }
    }
  }
}

template <class T, int D>
hipError_t launch_bwd(BwdArgs A, hipStream_t st) {
  constexpr bool kBf16 = std::is_same<T, uint16_t>::value;
  const int64_t rows = static_cast<int64_t>(A.B) * A.Hq * A.S;
  const int n_kt = (A.S + KB - 1) / KB;
  if constexpr (kBf16) {
    return launch_bf16_kernels(A, D, st);         // (delta comes from the dQ kernel)
  } else {
    hipLaunchKernelGGL((delta_kernel<T, D>), dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0, st, A);
    hipLaunchKernelGGL((dq_kernel<T, D>), dim3(A.B * A.Hkv * A.n_hg * A.n_qt), dim3(BT), 0, st, A);
    hipLaunchKernelGGL((dkdv_band_kernel<T, D>), dim3(A.B * A.Hkv * n_kt), dim3(BT), 0, st, A, n_kt);
    // twice the resident workgroups (one per CU: register bound) on 256 CUs
    const int n_qc = (A.S + QCH - 1) / QCH;
    const int BH = A.B * A.Hkv;
    const int nslots = BH >= 512 ? 1 : 512 / BH;
    hipLaunchKernelGGL((dkdv_glob_kernel<T, D>), dim3(BH * nslots), dim3(BT), 0, st, A, n_qc, nslots);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_prefill_backward(const void* q, const void* k, const void* v, const void* out,
                                   const void* dout, const float* lse, int dtype, int B, int Hq, int Hkv,
                                   int S, int D, const uint8_t* is_sep, const int32_t* rank,
                                   const int32_t* sep_pos, int a, int n, float scale, float* delta, float* dq,
                                   float* dk, float* dv, hipStream_t st) {
  BwdArgs A;
  A.q = q;
  A.k = k;
  A.v = v;
  A.out = out;
  A.dout = dout;
  A.lse = lse;
  A.is_sep = is_sep;
  A.rank = rank;
  A.sep_pos = sep_pos;
  A.delta = delta;
  A.dq = dq;
  A.dk = dk;
  A.dv = dv;
  A.B = B;
  A.Hq = Hq;
  A.Hkv = Hkv;
  A.S = S;
  A.a = a;
  A.n = n;
  A.G = Hq / Hkv;
  A.scale = scale;
  A.scale_log2 = scale * kLog2e;
  A.HPW = (A.G % 4 == 0) ? 4 : ((A.G % 2 == 0) ? 2 : 1);
  A.n_hg = A.G / A.HPW;
  A.QT = 32 * (BW / A.HPW);
  A.n_qt = (S + A.QT - 1) / A.QT;
  if (dtype == SEP_BF16)
    return D == 128 ? launch_bwd<uint16_t, 128>(A, st) : launch_bwd<uint16_t, 64>(A, st);
  return D == 128 ? launch_bwd<float, 128>(A, st) : launch_bwd<float, 64>(A, st);
}

}  // namespace sep
