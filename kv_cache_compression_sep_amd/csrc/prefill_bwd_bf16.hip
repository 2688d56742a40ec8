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

// The LDS byte address of a tile, hidden from the compiler's address
// arithmetic (which otherwise rebuilds every operand address of a tile from
// the ring's loop-carried pieces): each address below is then one add.
typedef __attribute__((address_space(3))) const char* lds_cptr;
__device__ __forceinline__ uint32_t tile_base(const char* p) {
  uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cptr)p));
  asm volatile("" : "+s"(a));
  return a;
}
__device__ __forceinline__ lds_cptr lds_at(uint32_t a) { return (lds_cptr)static_cast<uintptr_t>(a); }

// Helpers of the LDS-DMA tile loads (global_load_lds: no register results).
__device__ __forceinline__ void bw_fence() { asm volatile("" ::: "memory"); }

// A workgroup barrier for LDS hand-offs only: it waits for this wave's LDS
// accesses (lgkmcnt(0)) but not for its global stores and atomics, which
// may complete in the background.
__device__ __forceinline__ void lds_barrier() {
  bw_fence();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  bw_fence();
}

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
// 4 l); base and lds_base wave-uniform (taken from the first lane, so that
// they sit in scalar registers even where the compiler cannot prove them
// uniform). M0 carries the LDS base; these kernels make no other use of M0.
__device__ __forceinline__ const void* bw_uniform(const void* p) {
  const uint64_t v = reinterpret_cast<uintptr_t>(p);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  return reinterpret_cast<const void*>(static_cast<uintptr_t>(lo | (hi << 32)));
}
__device__ __forceinline__ void bw_dma16(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(bw_uniform(base)), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory", "m0");
}
__device__ __forceinline__ void bw_dma4(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(bw_uniform(base)), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory", "m0");
}

// Position of a query tile in a key block's sequence: query tile q of head h
// of the group, advanced one tile at a time (no divisions in the loop).
// Loop state that is uniform by construction, pinned to scalar registers:
// left to itself the compiler may keep it in VGPRs, and then every address
// derived from it costs VALU work and a readfirstlane per DMA.
__device__ __forceinline__ int bw_sgpr(int x) { return __builtin_amdgcn_readfirstlane(x); }

struct TileSeq {
  int h, q;
  __device__ void next(int ntq) {
    if (++q == ntq) {
      q = 0;
      ++h;
    }
    h = bw_sgpr(h);
    q = bw_sgpr(q);
  }
};

// ---------------------------------------------------------------- dQ (bf16)
// The forward's work items; the key tiles of 64 (gathered rows: initial and
// separator keys, then the band) land in a two-stage LDS ring by LDS-DMA one
// tile ahead (issued while the tile before is computed), their indices two
// tiles ahead.
template <int D>
__global__ void __launch_bounds__(BT, 2) dq_bf16_kernel(BwdArgs P) {
  using G = BGeo<D>;
  constexpr int CPR = G::CPR, KS = G::KS, DB = G::DB;
  constexpr int TILEB = KTQ * D * 2;
  constexpr int NINS = TILEB / 1024;              // 1 KB DMA ops per tensor and tile
  constexpr int PERW = NINS / BW;
  static_assert(NINS % BW == 0, "whole DMA ops per wave");
  static_assert(kWave % CPR == 0, "a wave's 16-byte slots span whole rows");
  __shared__ __attribute__((aligned(1024))) char kring[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) char vring[2 * TILEB];
  __shared__ int32_t idxbuf[3][KTQ];
  __shared__ uint64_t sepbits[3];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
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

  const int32_t* rk = P.rank + static_cast<int64_t>(b) * (S + 1);
  const int32_t* sp = P.sep_pos + static_cast<int64_t>(b) * S;
  const uint8_t* fl = P.is_sep + static_cast<int64_t>(b) * S;
  const TileInfo ti = tile_info<KTQ>(rk, S, P.a, P.n, q0, q1);
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(P.k) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(P.v) + static_cast<int64_t>(b * P.Hkv + g) * S * D;

  // wave 0: the key rows and separator flags of tile t (the entries of
  // tile_key), in two steps: index_load issues one load per lane from a
  // clamped, always valid address (no per-lane branch, so nothing waits for
  // it), index_write selects from what it returned and fills the index ring
  auto index_load = [&](int t) -> int {
    if (t < ti.ntg) return sp[min(max(ti.rank_a + t * KTQ + lane - ti.n_init, 0), S - 1)];
    return fl[min(ti.band_lo + (t - ti.ntg) * KTQ + lane, S - 1)];
  };
  auto index_write = [&](int t, int raw) {
    int key;
    bool f = false;
    if (t < ti.ntg) {                             // gathered: initial keys, then separators
      const int gu = t * KTQ + lane;
      key = gu >= ti.n_glob ? 0 : (gu < ti.n_init ? gu : raw);
    } else {                                      // band: consecutive keys and their flags
      const int j = ti.band_lo + (t - ti.ntg) * KTQ + lane;
      key = min(j, S - 1);
      f = j < S && raw != 0;
    }
    const uint64_t bits = ballot(f);
    idxbuf[t % 3][lane] = key;
    if (lane == 0) sepbits[t % 3] = bits;
  };
  const uint32_t k_lds = tile_base(kring);
  const uint32_t v_lds = tile_base(vring);
  auto issue = [&](int t) {                       // the DMA ops of tile t into stage t % 2
    const uint32_t st = (t & 1) * TILEB;
    // this lane's row and byte column in each op (the LDS chunk swizzle goes
    // into the global offsets), recomputed from an opaque copy of the lane
    // index each tile rather than held in registers through the loop
    int l = lane;
    asm volatile("" : "+v"(l));
    // the index reads first: a DMA (an opaque memory access) would keep a
    // later LDS read behind it, one round trip per op
    int key[PERW];
#pragma unroll
    for (int i = 0; i < PERW; ++i) key[i] = idxbuf[t % 3][(wave * PERW + i) * (kWave / CPR) + l / CPR];
#pragma unroll
    for (int i = 0; i < PERW; ++i) {
      const int r = (wave * PERW + i) * (kWave / CPR) + l / CPR;
      const uint32_t col = 16 * ((l % CPR) ^ G::swz(r));
      const uint32_t off = static_cast<uint32_t>(key[i]) * (D * 2) + col;
      const uint32_t dst = st + (wave * PERW + i) * 1024;
      bw_dma16(kb, off, k_lds + dst);
      bw_dma16(vb, off, v_lds + dst);
    }
  };
  // Wave 0's index loads of tiles 0 and 1 go out before the row loads of
  // Q, dO and out, so that its wait for them (which the compiler counts
  // exactly) does not include those, and tile 0's DMA is issued while the
  // rows are still landing.
  int ix0, ix1;                                   // (read only where loaded)
  if (wave == 0) {
    if (ti.ntiles > 0) ix0 = index_load(0);
    if (ti.ntiles > 1) ix1 = index_load(1);
  }
  // Q^T and dO^T fragments of this lane's query: d = 16 ks + 8 (lane / 32) + i,
  // and its out row for delta
  bf16x8 qf[KS], of[KS], ov[KS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(P.q) + (hrow + qc) * D + 8 * hsel;
    const uint16_t* dp = reinterpret_cast<const uint16_t*>(P.dout) + (hrow + qc) * D + 8 * hsel;
    const uint16_t* op = reinterpret_cast<const uint16_t*>(P.out) + (hrow + qc) * D + 8 * hsel;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks));
      of[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dp + 16 * ks));
      ov[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(op + 16 * ks));
    }
  }
  const float lse2 = P.lse[hrow + qc] * kLog2e;
  if (wave == 0) {
    if (ti.ntiles > 0) index_write(0, ix0);
    if (ti.ntiles > 1) index_write(1, ix1);
  }
  __syncthreads();
  if (ti.ntiles > 0) issue(0);
  // delta of this lane's query row, rowsum(dO o out) in fp32 (the two
  // halves of d sit in lanes l and l + 32); stored for the dK/dV kernels,
  // which run after this one
  float dlt = 0.0f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) dlt += static_cast<float>(of[ks][e]) * static_cast<float>(ov[ks][e]);
  dlt += __shfl_xor(dlt, 32);
  if (hsel == 0 && qi < S) P.delta[hrow + qi] = dlt;

  int toff[DB][2];
  tr_offsets<D>(lane, toff);
  f32x16 dacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dacc[db] = f32x16{};

  // the products of tile t (band tiles no row of the wave sees are skipped)
  auto tile_products = [&](int t) {
    const char* kst = kring + (t & 1) * TILEB;
    const char* vst = vring + (t & 1) * TILEB;
    const bool band = t >= ti.ntg;
    const int jmin = band ? ti.band_lo + (t - ti.ntg) * KTQ : 0;
    const int nvalid = band ? KTQ : min(KTQ, ti.n_glob - t * KTQ);
    if (band && (jmin > qmax || qw0 >= S)) return;
    const bool need_mask = band ? !(jmin + KTQ - 1 <= qw0 && jmin >= qmax - P.n + 1) : nvalid < KTQ;
    const uint64_t vis =
        need_mask ? (vis_word(band, qi, jmin, P.n, P.a, sepbits[t % 3], nvalid) >> (4 * hsel)) : ~0ull;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      // the K rows' operands; each V row operand is read into the registers
      // of the K operand that the S chain has just consumed, so that the V
      // reads are in flight during the S chain without a second set of
      // operand registers
      bf16x8 a[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[ks] = row_operand<D>(kst, 32 * mb + lane % 32, ks, lane);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sc = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sc = mfma32x32x16(a[ks], qf[ks], sc);
        a[ks] = row_operand<D>(vst, 32 * mb + lane % 32, ks, lane);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dp = mfma32x32x16(a[ks], of[ks], dp);
      __builtin_amdgcn_sched_barrier(0);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(__builtin_fmaf(sc[r], P.scale_log2, -lse2));
      if (need_mask) {                            // hidden pairs: P = +0 (AND with the sign-extended bit)
        const uint32_t word = static_cast<uint32_t>(vis >> (32 * mb));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t keep = __builtin_amdgcn_sbfe(word, 8 * (r / 4) + (r % 4), 1);
          uint32_t pb;                            // (the compiler would make the AND a compare and select)
          asm("v_and_b32 %0, %1, %2" : "=v"(pb) : "v"(__builtin_bit_cast(uint32_t, ds[r])), "v"(keep));
          ds[r] = __builtin_bit_cast(float, pb);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] *= dp[r] - dlt;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kcl = 0; kcl < 2; ++kcl) {
        const bf16x8 bds = pack8(ds + 8 * kcl);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dacc[db] = mfma32x32x16(tr_operand<D>(kst, toff[db], 2 * mb + kcl), bds, dacc[db]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int i = 0; i < 2 * DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One barrier per tile. Before it each wave waits for all of its loads:
  // its parts of tile t (issued during tile t - 1) and, on wave 0, the index
  // loads (its index writes complete too: lgkmcnt(0)). Past it, tile t is
  // published, and every wave is done with tile t - 1, whose stage then takes
  // tile t + 1 and whose index slot the indices of tile t + 2.
  for (int t = 0; t < ti.ntiles; ++t) {
    bw_fence();
    bw_wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    bw_fence();
    if (t + 1 < ti.ntiles) issue(t + 1);
    // wave 0 reads the indices of tile t + 2 now and writes them after this
    // tile's products, so that their global-memory latency is hidden behind
    // the MFMAs (the write waits for every load of the wave, the DMA of tile
    // t + 1 included, which has long landed by then)
    const bool nidx = wave == 0 && t + 2 < ti.ntiles;
    int nx;                                       // (read only where nidx holds: no default that
    if (nidx) nx = index_load(t + 2);             // would overwrite a load in flight)
    tile_products(t);
    if (nidx) index_write(t + 2, nx);
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
// query row), and each wave holds one of K^T, V^T in registers (the dS wave
// V^T negated: its product, started from delta, gives delta - dP at no VALU
// cost).
template <int D>
struct KVGeo {
  static constexpr int KS = D / 16;               // 16-wide k-steps over d
  static constexpr int DB = D / 32;               // 32-row d blocks
  static constexpr int NWAVE = 8;
  static constexpr int NTH = NWAVE * kWave;
};

// This lane's LDS byte offsets within a 32-row tile: the row reads of
// tile_scores (chunk 2 ks + lane / 32 of row lane % 32) and the transpose
// reads of tile_accumulate. Kept in registers, so that each operand address
// of a tile is one add to the tile's base.
template <int D>
struct LaneOff {
  uint32_t row[D / 16];
  int tr[D / 32][2];
  __device__ explicit LaneOff(int lane) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) row[ks] = 16 * BGeo<D>::slot(lane % 32, 2 * ks + lane / 32);
    tr_offsets<D>(lane, tr);
  }
};

// acc plus the KS products over d of tile rows lane % 32 with the register
// fragments b (one key per lane): all A operands are read before the first
// MFMA, so that the LDS latency is paid once per tile.
template <int D>
__device__ __forceinline__ f32x16 tile_scores(const char* tile, const LaneOff<D>& lo, const bf16x8 (&b)[D / 16],
                                              f32x16 acc = f32x16{}) {
  constexpr int KS = D / 16;
  bf16x8 a[KS];
  const uint32_t base = tile_base(tile);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    a[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<__attribute__((address_space(3))) const u32x4*>(
                                           lds_at(base + lo.row[ks])));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) acc = mfma32x32x16(a[ks], b[ks], acc);
  return acc;
}

// acc[db] += tile^T w over the 32 tile rows, per d block: the A operands
// come from the transpose reads, the B operands w[kc] hold the weights of
// accumulator elements 8 kc .. 8 kc + 7 (rows 16 kc .. 16 kc + 15).
template <int D>
__device__ __forceinline__ void tile_accumulate(const char* tile, const LaneOff<D>& lo, const bf16x8 (&w)[2],
                                                f32x16 (&acc)[D / 32]) {
  constexpr int DB = D / 32;
  bf16x8 a[2][DB];
  const uint32_t base = tile_base(tile);
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      constexpr int RB = BGeo<D>::CPR * 16;       // bytes per row
      const v4i16b x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16b*)(lds_at(base + lo.tr[db][0]) + 16 * kc * RB));
      const v4i16b x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16b*)(lds_at(base + lo.tr[db][1]) + 16 * kc * RB));
      const v8i16b cat = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      a[kc][db] = __builtin_bit_cast(bf16x8, cat);
    }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = mfma32x32x16(a[kc][db], w[kc], acc[db]);
}

// P wave, one query tile: bit il of vm says that tile row il is visible to
// this lane's key; masked false promises that every bit of every lane is
// set (a uniform branch skips the masking). P goes to pw[i * 64] (i < 4,
// elements 4 i .. 4 i + 3), hidden pairs as +0 (an AND with the pair's
// sign-extended bit).
template <int D>
__device__ __forceinline__ void p_tile(const char* Qs, const char* Os, const float* lse, const bf16x8 (&kf)[D / 16],
                                       const LaneOff<D>& lo, float scale_log2, int lane, uint32_t vm, bool masked,
                                       f32x4* pw, f32x16 (&dv)[D / 32]) {
  const int hsel = lane / 32;
  f32x4 l4[4];                                    // lse of rows 8 i + 4 (lane / 32) + e
#pragma unroll
  for (int i = 0; i < 4; ++i) l4[i] = *reinterpret_cast<const f32x4*>(lse + 8 * i + 4 * hsel);
  const f32x16 sc = tile_scores<D>(Qs, lo, kf);
  float p[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) p[r] = fast_exp2(__builtin_fmaf(sc[r], scale_log2, -l4[r / 4][r % 4] * kLog2e));
  if (masked) {
    const uint32_t vh = vm >> (4 * hsel);         // bit 8 (r / 4) + r % 4: accumulator element r
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t keep = __builtin_amdgcn_sbfe(vh, 8 * (r / 4) + (r % 4), 1);
      uint32_t pb;                                // (the compiler would make the AND a compare and select)
      asm("v_and_b32 %0, %1, %2" : "=v"(pb) : "v"(__builtin_bit_cast(uint32_t, p[r])), "v"(keep));
      p[r] = __builtin_bit_cast(float, pb);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) pw[i * kWave] = f32x4{p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]};
  const bf16x8 w[2] = {pack8(p), pack8(p + 8)};
  tile_accumulate<D>(Os, lo, w, dv);
}

// dS wave, the tile whose P the P wave left at pr; dm = delta - dP of its
// rows (the dP product run from an accumulator that starts at delta, with
// V negated), so dS = P (dP - delta) = -(P dm).
template <int D>
__device__ __forceinline__ void ds_tile(const char* Qs, const f32x4* pr, const f32x16& dm, const LaneOff<D>& lo,
                                        f32x16 (&dk)[D / 32]) {
  float ds[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 pq = pr[i * kWave];
#pragma unroll
    for (int e = 0; e < 4; ++e) ds[4 * i + e] = -(pq[e] * dm[4 * i + e]);
  }
  const bf16x8 w[2] = {pack8(ds), pack8(ds + 8)};
  tile_accumulate<D>(Qs, lo, w, dk);
}

// delta of the tile's rows in the accumulator layout (element r: row
// 8 (r / 4) + 4 (lane / 32) + r % 4)
__device__ __forceinline__ f32x16 rows_acc(const float* v, int lane) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(v + 8 * i + 4 * (lane / 32));
#pragma unroll
    for (int e = 0; e < 4; ++e) r[4 * i + e] = x[e];
  }
  return r;
}

// Bits [lo, hi) of a 32-row tile, the bounds clamped to the tile.
__device__ __forceinline__ uint32_t row_range(int lo, int hi) {
  lo = min(max(lo, 0), 32);
  hi = min(max(hi, lo), 32);
  return static_cast<uint32_t>((1ull << hi) - (1ull << lo));
}

// Query tiles of 32 rows (Q, dO, lse, delta) stream into a ring of NST LDS
// stages by LDS-DMA (global_load_lds: no register results), AHEAD tiles
// ahead of the one being computed. The NW issuing waves (waves 0 .. NW - 1)
// each issue exactly OPS DMA ops per tile (dummies into their junk row past
// the last tile, or for the lse/delta rows that only wave 0 loads), so one
// exact vmcnt count per tile says that a wave's own parts of tile t landed;
// a plain barrier then publishes the tile to every wave.
// Rows are placed with the swizzle of BGeo through the global offsets.
// The LDS byte address of p, computed once (wave-uniform).
__device__ __forceinline__ uint32_t lds_u32(const char* p) { return tile_base(p); }

// The dS wave reads tile t - 1 while tile t + AHEAD lands, and a wave may
// still read tile t - 2 when another issues tile t + AHEAD (one barrier per
// tile): NST = AHEAD + 3. Stages are named by index (0 .. NST - 1); the DMA
// geometry of this lane is computed once.
template <int D, int NW>
struct QRing {
  static constexpr int CPR = BGeo<D>::CPR;
  static constexpr int TB = QB * D * 2;           // bytes of a 32-row Q (or dO) tile
  static constexpr int NINS = TB / 1024;          // 1 KB DMA instructions per tensor
  static constexpr int PERW = NINS >= NW ? NINS / NW : 1;   // per wave (dummies past NINS)
  static constexpr int OPS = 2 * PERW + 2;        // + one dword op each for lse and delta
  static constexpr int AHEAD = 3;
  static constexpr int NST = AHEAD + 3;
  static constexpr int STAGE = 2 * TB + 2 * 64 * 4;
  static constexpr int BYTES = NST * STAGE;
  static_assert(NINS % NW == 0 || NINS < NW, "whole instructions per wave");
  char* ring;                                     // NST x [Q | dO | lse (64) | delta (64)]
  uint32_t ring_lds;                              // LDS address of the ring
  uint32_t junk_lds;                              // this wave's 1 KB junk row, target of dummy ops
  int wave;
  int row[PERW];                                  // this lane's tile row and byte column, per op
  uint32_t col[PERW];
  __device__ QRing(char* ring_, char* junk) : ring(ring_) {
    const int lane = threadIdx.x % kWave;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    ring_lds = lds_u32(ring_);
    junk_lds = lds_u32(junk) + wave * 1024;
#pragma unroll
    for (int i = 0; i < PERW; ++i) {
      const int sl = (wave * PERW + i) * kWave + lane;
      row[i] = sl / CPR;
      col[i] = 16 * ((sl % CPR) ^ BGeo<D>::swz(row[i]));
    }
  }
  __device__ char* q(int st) const { return ring + st * STAGE; }
  __device__ char* o(int st) const { return q(st) + TB; }
  __device__ float* l(int st) const { return reinterpret_cast<float*>(q(st) + 2 * TB); }
  __device__ float* d(int st) const { return l(st) + 64; }
  // the DMA ops of one tile (rows qt0.. of query row block hrow) into stage
  // st, or dummies into the junk row (hrow must still be a valid row block)
  __device__ void issue(const BwdArgs& P, bool real, int64_t hrow, int qt0, int st) const {
    const int lane = threadIdx.x % kWave;
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(P.q) + hrow * D;
    const uint16_t* ob = reinterpret_cast<const uint16_t*>(P.dout) + hrow * D;
    const uint32_t sb = ring_lds + st * STAGE;
#pragma unroll
    for (int i = 0; i < PERW; ++i) {
      const int ins = wave * PERW + i;
      const bool rw = real && ins < NINS;
      const uint32_t off = rw ? static_cast<uint32_t>(min(qt0 + row[i], P.S - 1) * (D * 2)) + col[i] : 0u;
      bw_dma16(qb, off, rw ? sb + ins * 1024 : junk_lds);
      bw_dma16(ob, off, rw ? sb + TB + ins * 1024 : junk_lds);
    }
    const bool rl = real && wave == 0;
    const uint32_t offl = rl ? 4u * static_cast<uint32_t>(min(qt0 + lane % 32, P.S - 1)) : 0u;
    bw_dma4(P.lse + hrow, offl, rl ? sb + 2 * TB : junk_lds);
    bw_dma4(P.delta + hrow, offl, rl ? sb + 2 * TB + 256 : junk_lds);
  }
};

// P of the last two query tiles, per key group and lane: [2][4][4][64] f32x4.
constexpr int kPBytes = 2 * 4 * 4 * kWave * 16;
__device__ __forceinline__ f32x4* p_slot(char* pbuf, int t, int kg, int lane) {
  return reinterpret_cast<f32x4*>(pbuf) + ((t & 1) * 4 + kg) * 4 * kWave + lane;
}

// Run compute(t, st) for t = 0 .. nt, st the ring stage of tile t (t = nt:
// no tile, the dS waves' last step). The tiles are those of the sequence
// from s0 (ntq query tiles per head, the first at row qs0; hrow_of(h) the
// query row block of head h). Every global load and store of the workgroup
// issued before the call must be complete or unrelated to vmcnt ordering:
// the call starts with a full wait.
// One barrier per tile, after the wait for tile t: every wave that passes
// it at step t has finished compute(t - 1), and its LDS stores of compute(t
// - 1) are complete (the wait includes lgkmcnt(0)). So compute(t) may read
// what compute(t - 1) wrote, and the DMA of tile t + AHEAD, issued after the
// barrier of step t - 1, only overwrites the stage of tile t - 3, which no
// wave reads after compute(t - 2). ISSUE: this wave is one of the ring's
// issuing waves (the others only wait at the barriers).
template <bool ISSUE, class RG, class HRow, class Compute>
__device__ __forceinline__ void stream_query_tiles(const BwdArgs& P, const RG& R, int nt, TileSeq s0, int ntq,
                                                   int qs0, HRow hrow_of, Compute compute) {
  bw_fence();
  __builtin_amdgcn_s_waitcnt(0);
  bw_fence();
  const int64_t hrow0 = hrow_of(s0.h);
  TileSeq is = s0;                                // next tile to issue
  int ist = 0;                                    // its stage
  int left = nt;                                  // tiles not yet issued
  auto issue_next = [&]() {
    const bool real = left > 0;
    R.issue(P, real, real ? hrow_of(is.h) : hrow0, qs0 + is.q * QB, ist);
    if (real) is.next(ntq);
    left = bw_sgpr(left - 1);
    ist = bw_sgpr(ist + 1 == RG::NST ? 0 : ist + 1);
  };
  if (ISSUE) {
#pragma unroll
    for (int t = 0; t < RG::AHEAD; ++t) issue_next();
  }
  int st = 0;
  for (int t = 0; t <= nt; ++t) {
    bw_fence();
    if (ISSUE) {
      issue_next();
      bw_wait_vm<RG::AHEAD * RG::OPS>();          // this wave's parts of tile t landed
    } else {
      __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0): its LDS accesses of compute(t - 1) done
    }
    __builtin_amdgcn_s_barrier();
    bw_fence();
    compute(t, st);
    st = bw_sgpr(st + 1 == RG::NST ? 0 : st + 1);
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
// t, the dS wave on tile t - 1 (dS, dK) and tile t (dP). vis(qt0) gives the
// visibility mask of the tile at row qt0 for this lane's key; a tile that
// no lane of the group sees is skipped by both waves alike. The two roles
// run separate loops (with the same barriers), so that each is
// register-allocated alone. The P waves issue the query-tile DMA: the dS
// waves' steps are the longer ones, so they only wait at the barriers.
template <int D, class Ring, class HRow, class Vis>
__device__ __forceinline__ void pair_loop(const BwdArgs& P, const Ring& R, char* pbuf, int nt, TileSeq s0, int ntq,
                                          int qs0, HRow hrow_of, bool pwave, int kg, int lane,
                                          const bf16x8 (&kv)[D / 16], const LaneOff<D>& lo, Vis vis,
                                          f32x16 (&acc)[D / 32]) {
  TileSeq cs = s0;                                // tile t
  if (pwave) {
    stream_query_tiles<true>(P, R, nt, s0, ntq, qs0, hrow_of, [&](int t, int st) {
      if (t == nt) return;
      const uint32_t vm = vis(qs0 + cs.q * QB);
      cs.next(ntq);
      if (ballot(vm != 0u) == 0) return;
      p_tile<D>(R.q(st), R.o(st), R.l(st), kv, lo, P.scale_log2, lane, vm, ballot(vm != ~0u) != 0,
                p_slot(pbuf, t, kg, lane), acc);
    });
  } else {
    bf16x8 nv[D / 16];                            // -V^T: a sign flip per bf16
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      nv[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, kv[ks]) ^ 0x80008000u);
    f32x16 dm = {};                               // delta - dP of tile t - 1
    bool prev = false;                            // tile t - 1 seen by the group
    stream_query_tiles<false>(P, R, nt, s0, ntq, qs0, hrow_of, [&](int t, int st) {
      if (prev) {
        const int sp = st == 0 ? Ring::NST - 1 : st - 1;
        ds_tile<D>(R.q(sp), p_slot(pbuf, t - 1, kg, lane), dm, lo, acc);
      }
      prev = false;
      if (t < nt) {
        prev = ballot(vis(qs0 + cs.q * QB) != 0u) != 0;
        cs.next(ntq);
        if (prev) dm = tile_scores<D>(R.o(st), lo, nv, rows_acc(R.d(st), lane));
      }
    });
  }
}

template <int D>
__global__ void __launch_bounds__(KVGeo<D>::NTH, 1) dkdv_band_bf16_kernel(BwdArgs P, int n_kt) {
  using KG = KVGeo<D>;
  using Ring = QRing<D, 4>;                 // the P waves issue the query-tile DMA
  __shared__ __attribute__((aligned(1024))) char ringmem[Ring::BYTES];
  __shared__ __attribute__((aligned(1024))) char junkmem[KG::NWAVE * 1024];
  __shared__ __attribute__((aligned(16))) char pbuf[kPBytes];
  const Ring R{ringmem, junkmem};
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int kg = wave % 4;                        // key group
  const bool pwave = wave < 4;
  const int hsel = lane / 32;
  // workgroups are dealt to the 8 XCDs in turn: give each XCD a run of
  // consecutive key blocks, whose query windows overlap, to share its L2
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % 8, xk = blockIdx.x / 8;
  const int xq = nwg / 8, xr = nwg % 8;
  const int idx = xcd < xr ? xcd * (xq + 1) + xk : xr * (xq + 1) + (xcd - xr) * xq + xk;
  const int kt = idx % n_kt;
  const int bgi = idx / n_kt;
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
  const LaneOff<D> lo(lane);
  f32x16 acc[KG::DB];
#pragma unroll
  for (int db = 0; db < KG::DB; ++db) acc[db] = f32x16{};
  // query tiles of the keys' windows, [j0, j0 + KB - 1 + n) capped at S, per head
  const int64_t qend64 = static_cast<int64_t>(j0) + KB - 1 + P.n;
  const int qend = static_cast<int>(qend64 < S ? qend64 : S);
  const int ntq = (qend - j0 + QB - 1) / QB;
  const int nt = P.G * ntq;
  const int hi_j = own ? j + min(S - j, P.n) : 0;  // rows i with j <= i < j + n, i < S
  auto hrow_of = [&](int h) { return static_cast<int64_t>(b * P.Hq + g * P.G + h) * S; };
  auto vis = [&](int qt0) { return own ? row_range(j - qt0, hi_j - qt0) : 0u; };
  pair_loop<D>(P, R, pbuf, nt, TileSeq{0, 0}, ntq, j0, hrow_of, pwave, kg, lane, kv, lo, vis, acc);
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

// dK, dV of the initial and separator keys ("global" keys: the list of
// initial positions, then sep_pos). Key tile u holds list entries
// [128 u, 128 u + 128); it meets every query row from its first key's
// position on, per head of the group: G * ntq(u) steps of one 32-row query
// tile. The steps of a kv head, key tile by key tile, are cut into nslots
// equal ranges, one per workgroup; a workgroup adds its partial dK, dV to
// memory (fp32 atomics) once per key tile its range touches, so the
// accumulation over query rows stays in registers for whole ranges.
template <int D>
__global__ void __launch_bounds__(KVGeo<D>::NTH, 1) dkdv_glob_bf16_kernel(BwdArgs P, int nslots) {
  using KG = KVGeo<D>;
  using Ring = QRing<D, 4>;                 // the P waves issue the query-tile DMA
  constexpr int NTH = KG::NTH;
  constexpr int RED = KG::NWAVE * 32 * 64 * 4;    // one 64-column pass of every wave's partial
  constexpr int SM = Ring::BYTES + kPBytes;
  static_assert(RED <= SM, "the flush buffer aliases the ring and the P buffers");
  __shared__ __attribute__((aligned(1024))) char smem[SM];
  __shared__ __attribute__((aligned(1024))) char junkmem[KG::NWAVE * 1024];
  __shared__ int32_t kpos[KB];
  __shared__ int32_t wsum[KG::NWAVE];
  __shared__ int32_t start[2];                    // first key tile of the range, first step in it
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
  const int G = P.G;
  const int32_t* rk = P.rank + static_cast<int64_t>(b) * (S + 1);
  const int32_t* sp = P.sep_pos + static_cast<int64_t>(b) * S;
  const int ninit = min(P.a, S);
  const int rank_a = rk[ninit];
  const int n_gl = ninit + rk[S] - rank_a;        // global keys of the sequence
  auto entry_pos = [&](int e) { return e < ninit ? e : sp[rank_a + (e - ninit)]; };
  const int nqt = (S + QB - 1) / QB;
  const int nkt = (n_gl + KB - 1) / KB;
  auto ntq_of = [&](int u) { return nqt - entry_pos(KB * u) / QB; };

  // Query tiles per key tile, summed: each thread a segment of key tiles,
  // an exclusive scan over the threads.
  const int seg = (nkt + NTH - 1) / NTH;
  const int ub = min(tid * seg, nkt);
  const int ue = min(ub + seg, nkt);
  int local = 0;
  for (int u = ub; u < ue; ++u) local += ntq_of(u);
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  if (tid == 0) start[0] = -1;
  __syncthreads();
  int excl = incl - local;
  int tot_q = 0;
  for (int w = 0; w < KG::NWAVE; ++w) {
    if (w < wave) excl += wsum[w];
    tot_q += wsum[w];
  }
  const int64_t total = static_cast<int64_t>(G) * tot_q;
  const int64_t s0 = total * slot / nslots;
  const int64_t s1 = total * (slot + 1) / nslots;
  // the thread whose key tiles hold step s0 records where the range starts
  if (s0 < s1 && static_cast<int64_t>(G) * excl <= s0 && s0 < static_cast<int64_t>(G) * (excl + local)) {
    int64_t before = static_cast<int64_t>(G) * excl;
    int u = ub;
    for (;; ++u) {
      const int64_t su = static_cast<int64_t>(G) * ntq_of(u);
      if (s0 < before + su) break;
      before += su;
    }
    start[0] = u;
    start[1] = static_cast<int>(s0 - before);
  }
  __syncthreads();

  const int64_t kvrow = static_cast<int64_t>(b * P.Hkv + g) * S;
  const uint16_t* kvb =
      (pwave ? reinterpret_cast<const uint16_t*>(P.k) : reinterpret_cast<const uint16_t*>(P.v)) + kvrow * D;
  float* dst = (pwave ? P.dv : P.dk) + kvrow * D;
  const float f = pwave ? 1.0f : P.scale;
  const LaneOff<D> lo(lane);

  int u = __builtin_amdgcn_readfirstlane(start[0]);   // (LDS values are not known to be uniform)
  int k0 = __builtin_amdgcn_readfirstlane(start[1]);
  int64_t rem = s1 - s0;
  while (rem > 0) {
    const int qs0 = entry_pos(KB * u) / QB * QB;
    const int ntq = nqt - qs0 / QB;
    const int su = G * ntq;
    const int k1 = static_cast<int>(min(static_cast<int64_t>(su), k0 + rem));
    lds_barrier();                                // kpos and the tiles of the previous key tile are consumed
    for (int e = tid; e < KB; e += NTH) {
      const int ee = KB * u + e;
      kpos[e] = ee < n_gl ? entry_pos(ee) : -1;
    }
    lds_barrier();
    const int j = kpos[32 * kg + lane % 32];      // this lane's key, -1 past the list
    bf16x8 kv[KG::KS];
    load_key_bf16<D>(kvb, j < 0 ? 0 : j, lane, kv);
    f32x16 acc[KG::DB];
#pragma unroll
    for (int db = 0; db < KG::DB; ++db) acc[db] = f32x16{};
    auto hrow_of = [&](int h) { return static_cast<int64_t>(b * P.Hq + g * G + h) * S; };
    auto vis = [&](int qt0) { return j >= 0 ? row_range(j - qt0, S - qt0) : 0u; };   // rows i >= j, i < S
    pair_loop<D>(P, R, pbuf, k1 - k0, TileSeq{k0 / ntq, k0 % ntq}, ntq, qs0, hrow_of, pwave, kg, lane, kv, lo,
                 vis, acc);
    // Add the partials with fp32 atomics, key row by key row through LDS, so
    // that each atomic instruction covers 2 x 32 consecutive floats of two
    // rows (2 cache lines) instead of one float of 32 rows; 64 columns a pass.
    // The barriers here order the LDS staging only: nothing waits for the
    // atomics until the next key tile's query stream (which starts with a
    // full wait) or the end of the kernel.
#pragma unroll
    for (int h = 0; h < D / 64; ++h) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dl = 32 * db + 8 * (r / 4) + 4 * hsel + (r % 4);       // column within the pass
          red[(wave * 32 + lane % 32) * 64 + (dl ^ (lane % 32))] = acc[2 * h + db][r] * f;
        }
      lds_barrier();
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
      lds_barrier();
    }
    rem -= k1 - k0;
    k0 = 0;
    ++u;
  }
}

}  // namespace

hipError_t launch_bf16_kernels(const BwdArgs& A, int D, hipStream_t st) {
  const int n_kt = (A.S + KB - 1) / KB;
  const int BH = A.B * A.Hkv;
  const int nslots = BH >= 256 ? 1 : 256 / BH;   // one workgroup per CU (their LDS allows no more)
  if (D == 128) {
    hipLaunchKernelGGL((dq_bf16_kernel<128>), dim3(A.B * A.Hkv * A.n_hg * A.n_qt), dim3(BT), 0, st, A);
    hipLaunchKernelGGL((dkdv_band_bf16_kernel<128>), dim3(A.B * A.Hkv * n_kt), dim3(KVGeo<128>::NTH), 0, st, A,
                       n_kt);
    hipLaunchKernelGGL((dkdv_glob_bf16_kernel<128>), dim3(BH * nslots), dim3(KVGeo<128>::NTH), 0, st, A, nslots);
  } else {
    hipLaunchKernelGGL((dq_bf16_kernel<64>), dim3(A.B * A.Hkv * A.n_hg * A.n_qt), dim3(BT), 0, st, A);
    hipLaunchKernelGGL((dkdv_band_bf16_kernel<64>), dim3(A.B * A.Hkv * n_kt), dim3(KVGeo<64>::NTH), 0, st, A,
                       n_kt);
    hipLaunchKernelGGL((dkdv_glob_bf16_kernel<64>), dim3(BH * nslots), dim3(KVGeo<64>::NTH), 0, st, A, nslots);
  }
  return hipGetLastError();
}

}  // namespace bwd
}  // namespace sep
