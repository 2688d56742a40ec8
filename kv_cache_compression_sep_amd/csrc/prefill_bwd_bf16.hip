// sep_attn_prefill_backward for bf16 inputs: dQ, dK, dV on the bf16 MFMA.
//
// Gradients of the Sep-Attention prefill (SepLLM pages: P2 §1.2 scaled
// masked softmax; P1 "Training-SepLLM" trains through the same mask); the
// decomposition is that of prefill_bwd.hip (dq over the forward's work
// items, dK/dV of window keys per 128-key block, dK/dV of initial and
// separator keys per (chunk, key tile) item with atomics).
#include "prefill_bwd.hpp"

#include <type_traits>

namespace sep {
namespace bwd {
namespace {


// ================================================================ bf16 inputs
// The same three passes on the 32x32x16 bf16 MFMA (fp32 accumulation), as
// mixed-precision attention backward passes run: Q, K, V, dO enter as bf16;
// P (for dV) and dS (for dQ and dK) are rounded to bf16 for their products;
// scores, P, dP, dS and every accumulator are fp32.
//
// Tiles sit in LDS row-major, 16-byte chunks XOR-swizzled by the row so that
// both a plain row read (one chunk of 32 rows) and the LDS transpose read
// (ds_read_b64_tr_b16, 4 rows x 64 bytes per half wave) are free of bank
// conflicts. The transpose read gives the A operand of the products that sum over
// tile rows (dQ^T += K^T dS^T, dV^T += dO^T P, dK^T += Q^T dS): lane l gets
// the 8 rows {16 kc + 8 e + 4 (l / 32) + k : e < 2, k < 4} of d column
// 32 db + l % 32, and the B operand takes the same 8 rows of the accumulator
// the scores came from (lane l holds rows 8 (r / 4) + 4 (l / 32) + r % 4),
// so both sides sum over the same rows in the same order.
typedef short v4i16b __attribute__((ext_vector_type(4)));
typedef short v8i16b __attribute__((ext_vector_type(8)));

template <int D>
struct BGeo {
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int KS = D / 16;               // 16-wide k-steps over d
  static constexpr int DB = D / 32;               // 32-row d blocks
  // chunk XOR f(row): f takes 16 (8) distinct values over 16 consecutive rows
  // (a plain read of one chunk of 32 rows hits every bank once per 16 lanes)
  // and puts 4 consecutive rows in 4 different 64-byte groups (a transpose
  // read of 4 rows x 64 bytes per 32 lanes is conflict-free as well)
  __device__ static int swz(int r) {
    return CPR == 16 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
  __device__ static int slot(int r, int c) { return r * CPR + (c ^ swz(r)); }
};

__device__ __forceinline__ v4i16b read_tr16b(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16b*)p);
}

// Byte offsets of this lane's transpose reads in rows R and R + 8 of a
// 16-row group (the swizzle repeats every 16 rows), d block db.
template <int D>
__device__ __forceinline__ void tr_offsets_block(int lane, int db, int (&off)[2]) {
  using G = BGeo<D>;
  const int tg = lane / 16, tj = lane % 16;
  const int th = tg / 2, tdh = tg % 2;
  const int R = 4 * th + tj / 4;
  const int dcol = 32 * db + 16 * tdh + 4 * (tj % 4);
#pragma unroll
  for (int e = 0; e < 2; ++e) off[e] = 16 * G::slot(R + 8 * e, dcol / 8) + 2 * (dcol % 8);
}

template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int (&off)[D / 32][2]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) tr_offsets_block<D>(lane, db, off[db]);
}

// A operand over rows 16 kc .. 16 kc + 15 of a tile, d block db.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, const int (&off)[2], int kc) {
  constexpr int RB = BGeo<D>::CPR * 16;           // bytes per row
  const v4i16b x0 = read_tr16b(tile + off[0] + (16 * kc) * RB);
  const v4i16b x1 = read_tr16b(tile + off[1] + (16 * kc) * RB);
  const v8i16b cat = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  return __builtin_bit_cast(bf16x8, cat);
}

// A operand of a product over d: chunk 2 ks + (lane / 32) of row r.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const char* tile, int r, int ks, int lane) {
  return __builtin_bit_cast(bf16x8,
                            *reinterpret_cast<const u32x4*>(tile + 16 * BGeo<D>::slot(r, 2 * ks + lane / 32)));
}

// B operand from 8 consecutive fp32 accumulator entries, rounded to bf16.
__device__ __forceinline__ bf16x8 pack8(const float* x) {
  const u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, w);
}

// ---------------------------------------------------------------- dQ (bf16)
// The forward's work items; the key tiles of 64 stream through LDS with a
// one-tile register prefetch, their indices two tiles ahead.
template <int D>
__global__ void __launch_bounds__(BT, 1) dq_bf16_kernel(BwdArgs P) {
  using G = BGeo<D>;
  constexpr int CPR = G::CPR, KS = G::KS, DB = G::DB;
  constexpr int TILEB = KTQ * D * 2;
  constexpr int LOADS = KTQ * CPR / BT;
  __shared__ __attribute__((aligned(16))) char kst[TILEB];
  __shared__ __attribute__((aligned(16))) char vst[TILEB];
  __shared__ int32_t idxbuf[3][KTQ];
  __shared__ uint64_t sepbits[3];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int hsel = lane / 32;

  PrefillArgs W;
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
  const int64_t hrow = static_cast<int64_t>(b * P.Hq + h) * S;
  const int qi = qw0 + lane % 32;
  const int qc = min(qi, S - 1);

  // Q^T and dO^T fragments of this lane's query: d = 16 ks + 8 (lane / 32) + i
  bf16x8 qf[KS], of[KS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(P.q) + (hrow + qc) * D + 8 * hsel;
    const uint16_t* op = reinterpret_cast<const uint16_t*>(P.dout) + (hrow + qc) * D + 8 * hsel;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks));
      of[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(op + 16 * ks));
    }
  }
  const float lse2 = P.lse[hrow + qc] * kLog2e;
  const float dlt = P.delta[hrow + qc];

  const int32_t* rk = P.rank + static_cast<int64_t>(b) * (S + 1);
  const int32_t* sp = P.sep_pos + static_cast<int64_t>(b) * S;
  const uint8_t* fl = P.is_sep + static_cast<int64_t>(b) * S;
  const TileInfo ti = tile_info<KTQ>(rk, S, P.a, P.n, q0, q1);
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(P.k) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(P.v) + static_cast<int64_t>(b * P.Hkv + g) * S * D;

  auto index_store = [&](int t) {                // wave 0: key rows and separator bits of tile t
    bool band;
    const int key = tile_key<KTQ>(ti, sp, S, t, lane, &band);
    bool f = false;
    if (band) {
      const int j = ti.band_lo + (t - ti.ntg) * KTQ + lane;
      f = (j < S) && (fl[j] != 0);
    }
    const uint64_t bits = ballot(f);
    idxbuf[t % 3][lane] = key;
    if (lane == 0) sepbits[t % 3] = bits;
  };
  u32x4 kr[LOADS], vr[LOADS];
  auto load_rows = [&](int t) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = tid / CPR + i * (BT / CPR);
      const int64_t off = static_cast<int64_t>(idxbuf[t % 3][row]) * D + 8 * (tid % CPR);
      kr[i] = *reinterpret_cast<const u32x4*>(kb + off);
      vr[i] = *reinterpret_cast<const u32x4*>(vb + off);
    }
  };
  if (wave == 0) {
    if (ti.ntiles > 0) index_store(0);
    if (ti.ntiles > 1) index_store(1);
  }
  __syncthreads();
  if (ti.ntiles > 0) load_rows(0);

  int toff[DB][2];
  tr_offsets<D>(lane, toff);
  f32x16 dacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dacc[db] = f32x16{};

  for (int t = 0; t < ti.ntiles; ++t) {
    __syncthreads();                              // tile t - 1 consumed
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = tid / CPR + i * (BT / CPR);
      const int sl = G::slot(row, tid % CPR);
      *reinterpret_cast<u32x4*>(kst + 16 * sl) = kr[i];
      *reinterpret_cast<u32x4*>(vst + 16 * sl) = vr[i];
    }
    if (wave == 0 && t + 2 < ti.ntiles) index_store(t + 2);
    __syncthreads();                              // tile t and index t + 2 published
    if (t + 1 < ti.ntiles) load_rows(t + 1);      // in flight during tile t

    const bool band = t >= ti.ntg;
    const int jmin = band ? ti.band_lo + (t - ti.ntg) * KTQ : 0;
    const int nvalid = band ? KTQ : min(KTQ, ti.n_glob - t * KTQ);
    if (band && (jmin > qmax || qw0 >= S)) continue;
    const bool need_mask = band ? !(jmin + KTQ - 1 <= qw0 && jmin >= qmax - P.n + 1) : nvalid < KTQ;
    const uint64_t vis =
        need_mask ? (vis_word(band, qi, jmin, P.n, P.a, sepbits[t % 3], nvalid) >> (4 * hsel)) : ~0ull;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 sc = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sc = mfma32x32x16(row_operand<D>(kst, 32 * mb + lane % 32, ks, lane), qf[ks], sc);
        dp = mfma32x32x16(row_operand<D>(vst, 32 * mb + lane % 32, ks, lane), of[ks], dp);
      }
      const uint32_t word = static_cast<uint32_t>(vis >> (32 * mb));
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool on = (word >> (8 * (r / 4) + (r % 4))) & 1u;
        const float p = on ? fast_exp2(__builtin_fmaf(sc[r], P.scale_log2, -lse2)) : 0.0f;
        ds[r] = p * (dp[r] - dlt);
      }
#pragma unroll
      for (int kcl = 0; kcl < 2; ++kcl) {
        const bf16x8 bds = pack8(ds + 8 * kcl);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dacc[db] = mfma32x32x16(tr_operand<D>(kst, toff[db], 2 * mb + kcl), bds, dacc[db]);
      }
    }
  }
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

// ---------------------------------------------------------------- dK, dV (bf16)
// A workgroup holds 128 keys in 4 groups of 32 and gives each group two
// waves. The P wave (waves 0-3) computes S = Q K^T and P, accumulates
// dV^T += dO^T P over the whole of d, and leaves P (fp32) in LDS. The dS wave
// (waves 4-7) computes dP = dO V^T and, one query tile later, dS = P (dP -
// delta) from that P, and accumulates dK^T += Q^T dS over the whole of d. So
// every product and every element of P and dS is computed once per (key,
// query row), and each wave holds one of K^T, V^T in registers.
template <int D>
struct KVGeo {
  static constexpr int KS = D / 16;               // 16-wide k-steps over d
  static constexpr int DB = D / 32;               // 32-row d blocks
  static constexpr int NWAVE = 8;
  static constexpr int NTH = NWAVE * kWave;
};

// The KS products over d of tile rows lane % 32 with the register fragments
// b (one key per lane): all A operands are read before the first MFMA, so
// that the LDS latency is paid once per tile.
template <int D>
__device__ __forceinline__ f32x16 tile_scores(const char* tile, const bf16x8 (&b)[D / 16], int lane) {
  constexpr int KS = D / 16;
  bf16x8 a[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) a[ks] = row_operand<D>(tile, lane % 32, ks, lane);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) acc = mfma32x32x16(a[ks], b[ks], acc);
  return acc;
}

// acc[db] += tile^T w over the 32 tile rows, per d block: the A operands
// come from the transpose reads, the B operands w[kc] hold the weights of
// accumulator elements 8 kc .. 8 kc + 7 (rows 16 kc .. 16 kc + 15).
template <int D>
__device__ __forceinline__ void tile_accumulate(const char* tile, const int (&toff)[D / 32][2],
                                                const bf16x8 (&w)[2], f32x16 (&acc)[D / 32]) {
  constexpr int DB = D / 32;
  bf16x8 a[2][DB];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int db = 0; db < DB; ++db) a[kc][db] = tr_operand<D>(tile, toff[db], kc);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = mfma32x32x16(a[kc][db], w[kc], acc[db]);
}

// P wave, one query tile: bit il of vm says that tile row il is visible to
// this lane's key. P goes to pw[i * 64] (i < 4, elements 4 i .. 4 i + 3),
// hidden pairs as +0 (an AND with the pair's sign-extended bit).
template <int D>
__device__ __forceinline__ void p_tile(const char* Qs, const char* Os, const float* lse,
                                       const bf16x8 (&kf)[D / 16], const int (&toff)[D / 32][2],
                                       float scale_log2, int lane, uint32_t vm, f32x4* pw,
                                       f32x16 (&dv)[D / 32]) {
  const int hsel = lane / 32;
  const uint32_t vh = vm >> (4 * hsel);           // bit 8 (r / 4) + r % 4: accumulator element r
  const f32x16 sc = tile_scores<D>(Qs, kf, lane);
  float p[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int il = 8 * (r / 4) + 4 * hsel + (r % 4);                  // query row of element r
    const float e = fast_exp2(__builtin_fmaf(sc[r], scale_log2, -lse[il] * kLog2e));
    const uint32_t keep = __builtin_amdgcn_sbfe(vh, 8 * (r / 4) + (r % 4), 1);
    uint32_t pb;                                  // (the compiler would make the AND a compare and select)
    asm("v_and_b32 %0, %1, %2" : "=v"(pb) : "v"(__builtin_bit_cast(uint32_t, e)), "v"(keep));
    p[r] = __builtin_bit_cast(float, pb);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) pw[i * kWave] = f32x4{p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]};
  const bf16x8 w[2] = {pack8(p), pack8(p + 8)};
  tile_accumulate<D>(Os, toff, w, dv);
}

// dS wave, the tile whose P the P wave left at pr and whose dP is dp.
template <int D>
__device__ __forceinline__ void ds_tile(const char* Qs, const float* dlt, const f32x4* pr, const f32x16& dp,
                                        const int (&toff)[D / 32][2], int lane, f32x16 (&dk)[D / 32]) {
  const int hsel = lane / 32;
  float ds[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 pq = pr[i * kWave];
#pragma unroll
    for (int e = 0; e < 4; ++e) ds[4 * i + e] = pq[e] * (dp[4 * i + e] - dlt[8 * i + 4 * hsel + e]);
  }
  const bf16x8 w[2] = {pack8(ds), pack8(ds + 8)};
  tile_accumulate<D>(Qs, toff, w, dk);
}

// Bits [lo, hi) of a 32-row tile, the bounds clamped to the tile.
__device__ __forceinline__ uint32_t row_range(int lo, int hi) {
  lo = min(max(lo, 0), 32);
  hi = min(max(hi, lo), 32);
  return static_cast<uint32_t>((1ull << hi) - (1ull << lo));
}

// Query tiles of 32 rows (Q, dO, lse, delta) stream into a ring of NST LDS
// stages by LDS-DMA (global_load_lds: no register results), AHEAD tiles
// ahead of the one being computed. Every wave issues exactly OPS DMA ops per
// tile (dummies into its junk row past the last tile, or for the lse/delta
// rows that only wave 0 loads), so one exact vmcnt count per tile says that
// its own parts of tile t landed; a plain barrier then publishes the tile.
// Rows are placed with the swizzle of BGeo through the global offsets.
__device__ __forceinline__ void bw_fence() { asm volatile("" ::: "memory"); }

template <int N>
__device__ __forceinline__ void bw_wait_vm() {    // s_waitcnt vmcnt(N) lgkmcnt(0)
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

__device__ __forceinline__ uint32_t bw_lds(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// Lane l's 16 (or 4) bytes from base + off land at LDS lds_base + 16 l (or
// 4 l); base and lds_base wave-uniform. M0 carries the LDS base; these
// kernels make no other use of M0.
__device__ __forceinline__ void bw_dma16(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void bw_dma4(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(base), "s"(lds_base) : "memory", "m0");
}

// The dS wave reads tile t - 1 while tile t + AHEAD lands: NST = AHEAD + 2.
template <int D, int NW>
struct QRing {
  static constexpr int CPR = BGeo<D>::CPR;
  static constexpr int TB = QB * D * 2;           // bytes of a 32-row Q (or dO) tile
  static constexpr int NINS = TB / 1024;          // 1 KB DMA instructions per tensor
  static constexpr int PERW = NINS >= NW ? NINS / NW : 1;   // per wave (dummies past NINS)
  static constexpr int OPS = 2 * PERW + 2;        // + one dword op each for lse and delta
  static constexpr int AHEAD = 3;
  static constexpr int NST = AHEAD + 2;
  static constexpr int STAGE = 2 * TB + 2 * 64 * 4;
  static constexpr int BYTES = NST * STAGE;
  static_assert(NINS % NW == 0 || NINS < NW, "whole instructions per wave");
  char* ring;                                     // NST x [Q | dO | lse (64) | delta (64)]
  char* junk;                                     // NW x 1 KB, targets of dummy ops
  __device__ char* q(int t) const { return ring + (t % NST) * STAGE; }
  __device__ char* o(int t) const { return q(t) + TB; }
  __device__ float* l(int t) const { return reinterpret_cast<float*>(q(t) + 2 * TB); }
  __device__ float* d(int t) const { return l(t) + 64; }
  // the DMA ops of tile t (rows qt0.. of query row block hrow), or dummies
  __device__ void issue(const BwdArgs& P, bool real, int64_t hrow, int qt0, int t) const {
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(P.q) + hrow * D;
    const uint16_t* ob = reinterpret_cast<const uint16_t*>(P.dout) + hrow * D;
    char* jw = junk + wave * 1024;
#pragma unroll
    for (int i = 0; i < PERW; ++i) {
      const int ins = wave * PERW + i;
      const bool rw = real && ins < NINS;
      const int sl = ins * kWave + lane;
      const int r = sl / CPR;
      const int c = (sl % CPR) ^ BGeo<D>::swz(r);
      const uint32_t off = rw ? static_cast<uint32_t>(min(qt0 + r, P.S - 1) * (D * 2) + 16 * c) : 0u;
      bw_dma16(qb, off, __builtin_amdgcn_readfirstlane(bw_lds(rw ? q(t) + ins * 1024 : jw)));
      bw_dma16(ob, off, __builtin_amdgcn_readfirstlane(bw_lds(rw ? o(t) + ins * 1024 : jw)));
    }
    const bool rl = real && wave == 0;
    const uint32_t offl = rl ? 4u * static_cast<uint32_t>(min(qt0 + lane % 32, P.S - 1)) : 0u;
    bw_dma4(P.lse + hrow, offl, __builtin_amdgcn_readfirstlane(bw_lds(rl ? reinterpret_cast<char*>(l(t)) : jw)));
    bw_dma4(P.delta + hrow, offl, __builtin_amdgcn_readfirstlane(bw_lds(rl ? reinterpret_cast<char*>(d(t)) : jw)));
  }
};

// P of the last two query tiles, per key group and lane: [2][4][4][64] f32x4.
constexpr int kPBytes = 2 * 4 * 4 * kWave * 16;
__device__ __forceinline__ f32x4* p_slot(char* pbuf, int t, int kg, int lane) {
  return reinterpret_cast<f32x4*>(pbuf) + ((t % 2) * 4 + kg) * 4 * kWave + lane;
}

// Run compute(t) for t = 0 .. nt (t = nt: no tile, the dS waves' last step);
// tile(t) gives (hrow, qt0) of tile t < nt. Every global load and store of
// the workgroup issued before the call must be complete or unrelated to
// vmcnt ordering: the call starts with a full wait. LDS stores of compute(t)
// are complete before compute(t + 1) starts on any wave (the wait of the
// tile count includes lgkmcnt(0) and precedes the publishing barrier).
template <class RG, class TileOf, class Compute>
__device__ __forceinline__ void stream_query_tiles(const BwdArgs& P, const RG& R, int nt, TileOf tile,
                                                   Compute compute) {
  bw_fence();
  __builtin_amdgcn_s_waitcnt(0);
  bw_fence();
#pragma unroll
  for (int t = 0; t < RG::AHEAD; ++t) {
    int64_t hrow;
    int qt0;
    tile(t < nt ? t : 0, &hrow, &qt0);
    R.issue(P, t < nt, hrow, qt0, t);
  }
  for (int t = 0; t <= nt; ++t) {
    bw_fence();
    __builtin_amdgcn_s_barrier();                 // compute(t - 1) done by every wave
    bw_fence();
    {
      const int tn = t + RG::AHEAD;
      int64_t hrow;
      int qt0;
      tile(tn < nt ? tn : 0, &hrow, &qt0);
      R.issue(P, tn < nt, hrow, qt0, tn);
    }
    bw_wait_vm<RG::AHEAD * RG::OPS>();            // this wave's parts of tile t landed
    __builtin_amdgcn_s_barrier();
    bw_fence();
    compute(t);
  }
  bw_fence();
  __builtin_amdgcn_s_waitcnt(0);                  // no DMA still landing (dummies included)
  __syncthreads();
}

// K^T (or V^T) fragments of key j: d = 16 ks + 8 (lane / 32) + i
template <int D>
__device__ __forceinline__ void load_key_bf16(const uint16_t* base, int j, int lane, bf16x8 (&f)[D / 16]) {
  const int hsel = lane / 32;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    f[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + static_cast<int64_t>(j) * D + 16 * ks + 8 * hsel));
}

// The query tile loop of one wave of a key group's pair: the P wave on tile
// t, the dS wave on tile t - 1 (dS, dK) and tile t (dP). vis(t) gives the
// visibility mask of tile t for this lane's key; a tile that no lane of the
// group sees is skipped by both waves alike. The two roles run separate
// loops (with the same barriers), so that each is register-allocated alone.
template <int D, class Ring, class TileOf, class Vis>
__device__ __forceinline__ void pair_loop(const BwdArgs& P, const Ring& R, char* pbuf, int nt, TileOf tile,
                                          bool pwave, int kg, int lane, const bf16x8 (&kv)[D / 16],
                                          const int (&toff)[D / 32][2], Vis vis, f32x16 (&acc)[D / 32]) {
  if (pwave) {
    stream_query_tiles(P, R, nt, tile, [&](int t) {
      if (t == nt) return;
      const uint32_t vm = vis(t);
      if (ballot(vm != 0u) == 0) return;
      p_tile<D>(R.q(t), R.o(t), R.l(t), kv, toff, P.scale_log2, lane, vm, p_slot(pbuf, t, kg, lane), acc);
    });
  } else {
    f32x16 dp = {};
    stream_query_tiles(P, R, nt, tile, [&](int t) {
      if (t > 0 && ballot(vis(t - 1) != 0u) != 0)
        ds_tile<D>(R.q(t - 1), R.d(t - 1), p_slot(pbuf, t - 1, kg, lane), dp, toff, lane, acc);
      if (t < nt && ballot(vis(t) != 0u) != 0) dp = tile_scores<D>(R.o(t), kv, lane);
    });
  }
}

template <int D>
__global__ void __launch_bounds__(KVGeo<D>::NTH, 1) dkdv_band_bf16_kernel(BwdArgs P, int n_kt) {
  using KG = KVGeo<D>;
  using Ring = QRing<D, KG::NWAVE>;
  __shared__ __attribute__((aligned(1024))) char ringmem[Ring::BYTES];
  __shared__ __attribute__((aligned(1024))) char junkmem[KG::NWAVE * 1024];
  __shared__ __attribute__((aligned(16))) char pbuf[kPBytes];
  const Ring R{ringmem, junkmem};
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int kg = wave % 4;                        // key group
  const bool pwave = wave < 4;
  const int hsel = lane / 32;
  const int kt = blockIdx.x % n_kt;
  const int bgi = blockIdx.x / n_kt;
  const int g = bgi % P.Hkv;
  const int b = bgi / P.Hkv;
  const int S = P.S;
  const int j0 = kt * KB;
  const int j = j0 + 32 * kg + lane % 32;
  const int jc = min(j, S - 1);
  const uint8_t* fl = P.is_sep + static_cast<int64_t>(b) * S;
  const bool own = j < S && j >= P.a && fl[jc] == 0;    // initial and separator keys: dkdv_glob
  const int64_t kvrow = static_cast<int64_t>(b * P.Hkv + g) * S;
  bf16x8 kv[KG::KS];
  load_key_bf16<D>((pwave ? reinterpret_cast<const uint16_t*>(P.k) : reinterpret_cast<const uint16_t*>(P.v)) +
                       kvrow * D,
                   jc, lane, kv);
  int toff[KG::DB][2];
  tr_offsets<D>(lane, toff);
  f32x16 acc[KG::DB];
#pragma unroll
  for (int db = 0; db < KG::DB; ++db) acc[db] = f32x16{};
  // query tiles of the keys' windows, [j0, j0 + KB - 1 + n) capped at S, per head
  const int64_t qend64 = static_cast<int64_t>(j0) + KB - 1 + P.n;
  const int qend = static_cast<int>(qend64 < S ? qend64 : S);
  const int ntq = (qend - j0 + QB - 1) / QB;
  const int nt = P.G * ntq;
  const int hi_j = own ? j + min(S - j, P.n) : 0;  // rows i with j <= i < j + n, i < S
  auto tile = [&](int t, int64_t* hrow, int* qt0) {
    *hrow = static_cast<int64_t>(b * P.Hq + g * P.G + t / ntq) * S;
    *qt0 = j0 + (t % ntq) * QB;
  };
  auto vis = [&](int t) {
    const int qt0 = j0 + (t % ntq) * QB;
    return own ? row_range(j - qt0, hi_j - qt0) : 0u;
  };
  pair_loop<D>(P, R, pbuf, nt, tile, pwave, kg, lane, kv, toff, vis, acc);
  if (j < S) {
    float* dst = (pwave ? P.dv : P.dk) + (kvrow + j) * D;
    const float f = pwave ? 1.0f : P.scale;
#pragma unroll
    for (int db = 0; db < KG::DB; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * q + 4 * hsel) =
            f32x4{acc[db][4 * q] * f, acc[db][4 * q + 1] * f, acc[db][4 * q + 2] * f, acc[db][4 * q + 3] * f};
  }
}

template <int D>
__global__ void __launch_bounds__(KVGeo<D>::NTH, 1) dkdv_glob_bf16_kernel(BwdArgs P, int n_qc, int nslots) {
  using KG = KVGeo<D>;
  using Ring = QRing<D, KG::NWAVE>;
  constexpr int RED = KG::NWAVE * 32 * 64 * 4;    // one 64-column pass of every wave's partial
  constexpr int SM = Ring::BYTES + kPBytes;
  static_assert(RED <= SM, "the flush buffer aliases the ring and the P buffers");
  __shared__ __attribute__((aligned(1024))) char smem[SM];
  __shared__ __attribute__((aligned(1024))) char junkmem[KG::NWAVE * 1024];
  __shared__ int32_t kpos[KB];
  __shared__ int32_t tstart[kMaxChunks + 1];
  __shared__ int32_t wsum[KG::NWAVE];
  const Ring R{smem, junkmem};
  char* pbuf = smem + Ring::BYTES;
  // one wave's partial over 64 columns, key-major, column ^ key: [NWAVE][32][64]
  float* red = reinterpret_cast<float*>(smem);
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int kg = wave % 4;
  const bool pwave = wave < 4;
  const int hsel = lane / 32;
  const int BH = P.B * P.Hkv;
  const int bgi = blockIdx.x % BH;
  const int slot = blockIdx.x / BH;
  const int g = bgi % P.Hkv;
  const int b = bgi / P.Hkv;
  const int S = P.S;
  const int32_t* rk = P.rank + static_cast<int64_t>(b) * (S + 1);
  const int32_t* sp = P.sep_pos + static_cast<int64_t>(b) * S;
  const int ninit = min(P.a, S);
  const int rank_a = rk[ninit];
  auto n_global = [&](int c1) { return min(ninit, c1) + (c1 > ninit ? rk[c1] - rank_a : 0); };
  const int total = chunk_tile_prefix<KG::NTH>(n_global, S, n_qc, tstart, wsum);

  const int64_t kvrow = static_cast<int64_t>(b * P.Hkv + g) * S;
  const uint16_t* kvb =
      (pwave ? reinterpret_cast<const uint16_t*>(P.k) : reinterpret_cast<const uint16_t*>(P.v)) + kvrow * D;
  float* dst = (pwave ? P.dv : P.dk) + kvrow * D;
  const float f = pwave ? 1.0f : P.scale;
  int toff[KG::DB][2];
  tr_offsets<D>(lane, toff);

  for (int w = slot; w < total; w += nslots) {
    const int qc = chunk_of(tstart, n_qc, w);
    const int u0 = (w - tstart[qc]) * KB;
    const int c0 = qc * QCH;
    const int c1 = min(c0 + QCH, S);
    const int n_in = min(ninit, c1);
    const int n_gl = n_global(c1);
    __syncthreads();                              // kpos and the tiles of the previous item are consumed
    for (int u = tid; u < KB; u += KG::NTH) {
      const int uu = u0 + u;
      kpos[u] = uu >= n_gl ? -1 : (uu < n_in ? uu : sp[rank_a + (uu - n_in)]);
    }
    __syncthreads();
    const int j = kpos[32 * kg + lane % 32];      // this lane's key, -1 past the list
    bf16x8 kv[KG::KS];
    load_key_bf16<D>(kvb, j < 0 ? 0 : j, lane, kv);
    f32x16 acc[KG::DB];
#pragma unroll
    for (int db = 0; db < KG::DB; ++db) acc[db] = f32x16{};
    const int jlo = kpos[0];
    const int qs0 = max(c0, jlo) / QB * QB;
    const int ntq = (c1 - qs0 + QB - 1) / QB;
    const int nt = P.G * ntq;
    const int lo_j = max(c0, j);                  // rows i of the chunk [c0, c1) with i >= j
    auto tile = [&](int t, int64_t* hrow, int* qt0) {
      *hrow = static_cast<int64_t>(b * P.Hq + g * P.G + t / ntq) * S;
      *qt0 = qs0 + (t % ntq) * QB;
    };
    auto vis = [&](int t) {
      const int qt0 = qs0 + (t % ntq) * QB;
      return j >= 0 ? row_range(lo_j - qt0, c1 - qt0) : 0u;
    };
    pair_loop<D>(P, R, pbuf, nt, tile, pwave, kg, lane, kv, toff, vis, acc);
    // Add the partials with fp32 atomics, key row by key row through LDS, so
    // that each atomic instruction covers 2 x 32 consecutive floats of two
    // rows (2 cache lines) instead of one float of 32 rows; 64 columns a pass.
#pragma unroll
    for (int h = 0; h < D / 64; ++h) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dl = 32 * db + 8 * (r / 4) + 4 * hsel + (r % 4);       // column within the pass
          red[(wave * 32 + lane % 32) * 64 + (dl ^ (lane % 32))] = acc[2 * h + db][r] * f;
        }
      __syncthreads();
#pragma unroll 4
      for (int pass = 0; pass < 16; ++pass) {
        const int row = 2 * pass + lane / 32;
        const int jr = kpos[32 * kg + row];
        if (jr >= 0) {
#pragma unroll
          for (int e = 0; e < 2; ++e)
            atomicAdd(dst + static_cast<int64_t>(jr) * D + 64 * h + 32 * e + lane % 32,
                      red[(wave * 32 + row) * 64 + ((32 * e + lane % 32) ^ row)]);
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_bf16_kernels(const BwdArgs& A, int D, hipStream_t st) {
  const int n_kt = (A.S + KB - 1) / KB;
  const int n_qc = (A.S + QCH - 1) / QCH;
  const int BH = A.B * A.Hkv;
  const int nslots = BH >= 512 ? 1 : 512 / BH;   // twice the resident workgroups on 256 CUs
  if (D == 128) {
    hipLaunchKernelGGL((dq_bf16_kernel<128>), dim3(A.B * A.Hkv * A.n_hg * A.n_qt), dim3(BT), 0, st, A);
    hipLaunchKernelGGL((dkdv_band_bf16_kernel<128>), dim3(A.B * A.Hkv * n_kt), dim3(KVGeo<128>::NTH), 0, st, A,
                       n_kt);
    hipLaunchKernelGGL((dkdv_glob_bf16_kernel<128>), dim3(BH * nslots), dim3(KVGeo<128>::NTH), 0, st, A, n_qc,
                       nslots);
  } else {
    hipLaunchKernelGGL((dq_bf16_kernel<64>), dim3(A.B * A.Hkv * A.n_hg * A.n_qt), dim3(BT), 0, st, A);
    hipLaunchKernelGGL((dkdv_band_bf16_kernel<64>), dim3(A.B * A.Hkv * n_kt), dim3(KVGeo<64>::NTH), 0, st, A,
                       n_kt);
    hipLaunchKernelGGL((dkdv_glob_bf16_kernel<64>), dim3(BH * nslots), dim3(KVGeo<64>::NTH), 0, st, A, n_qc,
                       nslots);
  }
  return hipGetLastError();
}

}  // namespace bwd
}  // namespace sep
