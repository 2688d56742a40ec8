// sep_attn_prefill, bf16 path: Sep-Attention prefill on 32x32x16 bf16 MFMA.
//
// Work decomposition (prefill.hpp): a workgroup owns one query tile of the
// HPW query heads that share a key/value head, and walks its key list
// (gathered initial + separator keys, then the dense band) in tiles of 64
// keys. Eight waves (two per SIMD) each hold 32 query rows of one head, so
// every K/V tile staged in LDS feeds 8 x 32 query rows.
//
// Staging: K and V tiles go straight from global memory into LDS with
// 16-byte LDS-DMA loads (no registers), each into a ring of four stages.
// K of tile t + 3 and V of tile t + 2 are issued in iteration t, inside the
// wave's VALU phase (below), spread over its exponentials. Rows are
// stored row-major with the 16-byte chunk index XOR-swizzled by the row, one
// swizzle for K (the QK reads take one chunk of 32 rows) and one for V (a
// transposed read takes 64 bytes of 4 rows per half wave), so that both hit
// distinct banks. The data a tile's gather needs (its slice of sep_pos, or
// for band tiles two shifted slices of rank whose difference gives the
// separator bits) also arrives by LDS-DMA, seven tiles ahead, into an index
// ring; the gather entries of tile t + 4 are read from it in iteration t,
// one iteration before its rows are formed and its loads issued, so that no
// load address waits for LDS (LDS destinations are plain 32-bit offsets,
// computed on the scalar unit). So the key loop has no global load with a register result: every
// wait is explicit. Each wave issues exactly 1 + OPS loads per iteration (a
// fixed dummy address past the last tile), waits with one exact vmcnt for
// its own loads of K(t) and V(t - 1), and a plain barrier publishes them.
//
// Scores are computed transposed, S^T = K Q^T: each lane owns one query
// column, so a row max is a max over the lane's registers plus one exchange
// with lane l^32, and the exponentiated scores already sit in the B-operand
// layout of O^T = V^T P^T. The V^T A-operand is read with the LDS transpose
// load (ds_read_b64_tr_b16): pointing a 16-lane group at four consecutive key
// rows gives each lane four keys of one d column.
//
// Software pipeline: PV of tile t - 1 runs in iteration t (P kept packed in
// registers, V still in its stage), so an iteration splits into an MFMA-only
// phase (QK of tile t, PV of tile t - 1) and a VALU-only phase (mask and
// softmax of tile t). The two waves on a SIMD (waves w and w + 4) run the
// two phases in opposite order, so one wave's MFMAs overlap the other's VALU
// work. Softmax is online in fp32 in the log2 domain with lazy rescaling
// (the running max moves only when a row's max grows by more than 8); a move
// scales O and l just before the next PV. P is rounded to bf16 for the PV
// product, and l sums the same rounded values on the MFMA pipe (a block of
// ones as one more A operand).
#include "prefill.hpp"
#include "internal.hpp"

#include <type_traits>

namespace sep {
namespace {

constexpr int KT = 64;                 // keys per tile
constexpr int NW = 8;                  // waves per workgroup
constexpr int NT = NW * kWave;
constexpr int KSTAGES = 4;             // K ring depth (tiles)
constexpr int VSTAGES = 4;             // V ring depth (tiles)
constexpr int KAHEAD = 3;              // K of tile t + KAHEAD is issued in iteration t
constexpr int VAHEAD = 2;              // V of tile t + VAHEAD is issued in iteration t
constexpr int IAHEAD = 7;              // index slices loaded this many tiles ahead
constexpr int IDXR = 8;                // index ring depth (> IAHEAD)
static_assert(IDXR > IAHEAD && IAHEAD >= KAHEAD + 4, "index ring too shallow");
constexpr float kLazy = 8.0f;
constexpr int kOpsEnd = 1 << 16;       // the end of a wave's op range [lo, hi): past its last op
// V of tiles t - 1 .. t + VAHEAD and K of tiles t .. t + KAHEAD are live in
// iteration t
static_assert(KAHEAD < KSTAGES && VAHEAD + 2 <= VSTAGES, "ring too shallow for the pipeline");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

template <int D>
struct Geo {
  static constexpr int CPR = D / 8;                    // 16-byte chunks per row
  static constexpr int TB = KT * D * 2;                // bytes of one K (or V) tile
  static constexpr int INSTR = TB / 1024;              // wave-wide 1 KB loads per tile
  static constexpr int PER_WAVE = INSTR / NW;          // per wave, per tensor
  static constexpr int OPS = 2 * PER_WAVE;             // K + V LDS-DMA ops per wave per iteration
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static_assert(PER_WAVE >= 1, "tile too small for the wave count");
  // 16-byte slot of (row r, chunk c) in a K stage: the QK reads take one
  // chunk of 32 consecutive rows, so the chunk is XOR-ed with the row.
  __device__ static int swz_k(int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int slot(int r, int c) { return r * CPR + (c ^ swz_k(r)); }
  // ... and in a V stage: a transposed read covers 4 consecutive rows x 64
  // bytes per 32 lanes, so rows that share bank positions get their chunk
  // groups of four exchanged.
  __device__ static int swz_v(int r) { return CPR == 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
  __device__ static int slot_v(int r, int c) { return r * CPR + (c ^ swz_v(r)); }
};

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Wait until this wave's loads of K(t) and V(t - 1) landed (and its LDS
// reads of the previous iteration completed), then a plain barrier. Memory
// ops of a wave in issue order: the index slices of tiles 0..6, [full
// wait], K(0); K(1), V(0); K(2), V(1); then per iteration t: one index
// slice, K(t + 3), V(t + 2). Both K(t) and V(t - 1) are issued in
// iteration t - 3 (or the prologue), V last; the ops issued after them are
// t = 0: 2*OPS; t = 1: 2*OPS + 1; t >= 2: 2*OPS + 2. Loads complete in
// issue order.
template <int OPS>
__device__ __forceinline__ void tile_barrier(int t) {
  compiler_fence();
  if (t >= 2) wait_vm_lgkm0<2 * OPS + 2>();
  else if (t == 1) wait_vm_lgkm0<2 * OPS + 1>();
  else wait_vm_lgkm0<2 * OPS>();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// Asynchronous global -> LDS copies from a wave-uniform base address plus a
// per-lane 32-bit byte offset. Lane l's 16 (or 4) bytes land at LDS address
// lds_base + 16*l (or + 4*l); lds_base is wave-uniform. There is no register
// result, so nothing waits for them except the explicit vmcnt. M0 carries
// the LDS base; the kernel makes no other use of M0 (no LDS-DMA builtins, no
// message or GWS instructions), so setting it inside the asm statement
// cannot disturb compiler-generated code.
__device__ __forceinline__ void dma_x4(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void dma_x1(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(base), "s"(lds_base) : "memory", "m0");
}

__device__ __forceinline__ v4i16 read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
}

// -inf where bit `pos` of `word` is clear (branch-free: extract, then select bits)
__device__ __forceinline__ float mask_bit(float s, uint32_t word, int pos) {
  const uint32_t m = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(word), pos, 1));
  const uint32_t x = __builtin_bit_cast(uint32_t, s);
  return __builtin_bit_cast(float, (x & m) | (0xff800000u & ~m));
}

template <bool B>
using flag = std::integral_constant<bool, B>;

template <int D>
__global__ void __launch_bounds__(NT, 1) prefill_bf16_kernel(PrefillArgs P) {
  using G = Geo<D>;
  constexpr int CPR = G::CPR;
  constexpr int TB = G::TB;
  constexpr int KS = G::KS;
  constexpr int DB = G::DB;
  constexpr int PW = G::PER_WAVE;
  constexpr int OSTR = D + 8;                          // bf16 output-staging row stride
  static_assert(NW * 32 * OSTR * 2 <= (KSTAGES + VSTAGES) * TB, "output staging must fit the ring");

  __shared__ __attribute__((aligned(1024))) char ring[(KSTAGES + VSTAGES) * TB];   // K stages, then V stages
  __shared__ __attribute__((aligned(16))) int32_t idxr[IDXR][2][KT];   // index slices
  __shared__ __attribute__((aligned(16))) int32_t junk[NW][KT];       // dummy-load targets

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform

  int pair, qt;
  work_item(P, blockIdx.x, &pair, &qt);
  const int hg = pair % P.n_hg;
  const int bg = pair / P.n_hg;
  const int g = bg % P.Hkv;
  const int b = bg / P.Hkv;
  const int S = P.S;                                   // query rows
  const int Skv = P.Skv;                               // key rows (S, except in chunk mode)
  const int qv = P.q_base;                             // key index of query row 0
  const int q0 = qt * P.QT;
  const int q1 = min(q0 + P.QT, S);
  const int hw = wave % P.HPW;
  const int rb = wave / P.HPW;
  const int h = g * P.G + hg * P.HPW + hw;
  const int qw0 = q0 + 32 * rb;                        // this wave's first query row

  // ---- Q fragments first: their loads are in flight while rank is read
  //      and the first index slices land
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(P.q) + static_cast<int64_t>(b * P.Hq + h) * S * D;
  bf16x8 qf[KS];
  {
    const int qrow = min(qw0 + lane % 32, S - 1);
    const uint16_t* p = qb + static_cast<int64_t>(qrow) * D + 8 * (lane / 32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p + 16 * ks));
  }

  const int32_t* rk = P.rank + static_cast<int64_t>(b) * (Skv + 1);
  const int32_t* sp = P.sep_pos + static_cast<int64_t>(b) * Skv;
  const int key_lo = P.key_lo == nullptr ? 0 : P.key_lo[b];
  const TileInfo ti = tile_info<KT>(rk, Skv, P.a, P.n, qv + q0, qv + q1, key_lo);

  const char* kb = reinterpret_cast<const char*>(P.k) + static_cast<int64_t>(b * P.Hkv + g) * Skv * D * 2;
  const char* vb = reinterpret_cast<const char*>(P.v) + static_cast<int64_t>(b * P.Hkv + g) * Skv * D * 2;

  // ---- index slice of tile t into ring slot t % IDXR: wave 0 loads
  //      sep_pos entries (global tiles) or rank[jmin + u]; wave 1 loads
  //      rank[jmin + u + 1] (band tiles); the other waves, and every wave
  //      past the last tile, load one fixed word into their junk row.
  auto issue_index = [&](int t) {
    const bool real = t < ti.ntiles;
    const bool band = t >= ti.ntg;
    const int32_t* base = rk;                          // fixed dummy address
    uint32_t off = 0;
    // LDS addresses as 32-bit integers (no generic-pointer arithmetic)
    uint32_t dst = lds_addr(junk) + 4u * KT * wave;
    if (real && wave < 2) {
      if (!band) {
        if (wave == 0) {
          base = sp;
          off = 4u * min(max(ti.rank_a + t * KT + lane - ti.n_init, 0), Skv - 1);
          dst = lds_addr(idxr) + 4u * KT * 2 * (t % IDXR);
        }
      } else {
        off = 4u * min(ti.band_lo + (t - ti.ntg) * KT + lane + wave, Skv);
        dst = lds_addr(idxr) + 4u * KT * (2 * (t % IDXR) + wave);
      }
    }
    dma_x1(base, off, dst);
  };
  // the sep_pos entries this lane's rows of tile t would gather, from the
  // tile's index slice (read for every tile, used for gathered ones)
  auto read_gather = [&](int t, int (&g)[PW]) {
#pragma unroll
    for (int i = 0; i < PW; ++i) g[i] = idxr[t % IDXR][0][((wave * PW + i) * kWave + lane) / CPR];
  };
  // key rows this lane copies for tile t (row 0 past the last tile)
  auto rows_from = [&](int t, const int (&g)[PW], int (&rows)[PW]) {
    const bool real = t < ti.ntiles;
    const bool band = t >= ti.ntg;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int r = ((wave * PW + i) * kWave + lane) / CPR;
      int key;
      if (band) {
        key = min(ti.band_lo + (t - ti.ntg) * KT + r, Skv - 1);
      } else {
        const int u = t * KT + r;
        key = u < ti.n_init ? u : (u >= ti.n_glob ? 0 : g[i]);
      }
      rows[i] = real ? key : 0;
    }
  };
  auto rows_of = [&](int t, int (&rows)[PW]) {
    int g[PW];
    read_gather(t, g);
    rows_from(t, g, rows);
  };
  // ---- LDS-DMA of the K (or V) rows of tile t into its ring stage
  auto issue_rows = [&](const char* base, uint32_t stage0, int t, const int (&rows)[PW], auto is_v, int lo = 0, int hi = kOpsEnd) {
    const uint32_t st = stage0 + (t % (decltype(is_v)::value ? VSTAGES : KSTAGES)) * TB;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      if (i < lo || i >= (hi < PW ? hi : PW)) continue;
      const int ins = wave * PW + i;                   // 1 KB block of the tile
      const int sl = ins * kWave + lane;               // 16-byte slot this lane fills
      const int r = sl / CPR;
      const int pos = sl % CPR;
      const int c = pos ^ (decltype(is_v)::value ? G::swz_v(r) : G::swz_k(r));   // chunk for that slot
      const uint32_t off = static_cast<uint32_t>(rows[i]) * (D * 2) + 16u * c;
      dma_x4(base, off, st + ins * 1024);
    }
  };
  char* const kring = ring;
  char* const vring = ring + KSTAGES * TB;
  const uint32_t kring_lds = lds_addr(ring);
  const uint32_t vring_lds = kring_lds + KSTAGES * TB;

  for (int t = 0; t < IAHEAD; ++t) issue_index(t);
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0);                       // index slices 0..6 landed
  __syncthreads();
  // key rows of V(t + 2), and the gather entries of tile t + 3, read one
  // iteration before the rows are needed so that no LDS read is waited for
  // in the load issue
  int vrows[PW], graw[PW];
  {
    int r0[PW], r1[PW];
    rows_of(0, r0);
    issue_rows(kb, kring_lds, 0, r0, flag<false>{});
    rows_of(1, r1);
    issue_rows(kb, kring_lds, 1, r1, flag<false>{});
    issue_rows(vb, vring_lds, 0, r0, flag<true>{});
    rows_of(2, vrows);
    issue_rows(kb, kring_lds, 2, vrows, flag<false>{});
    issue_rows(vb, vring_lds, 1, r1, flag<true>{});
    read_gather(3, graw);
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  u32x4 pk[4];                                         // bf16 P of the previous tile, per 16-key chunk
  // l, the row sum of P, is accumulated by the MFMA pipe: O^T gets one more
  // 32-row block whose A operand is all ones, so every row of lacc holds
  // sum_k P[q, k] for the lane's query q, in the same scale as O
  f32x16 lacc = {};
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  float m_run = -INFINITY, corr = 1.0f;
  bool resc = false;
  const int qmax = qv + min(qw0 + 31, S - 1);          // key index of the wave's last query
  const int hsel = lane / 32;
  const int qrow = qw0 + lane % 32;                    // this lane's query row
  const int qi = qv + qrow;                            // and its key index
  const int qwv0 = qv + qw0;

  // per-lane LDS byte offsets of the QK reads (chunk 2*ks + hsel of rows
  // lane%32 [+32]) and of the transposed V reads (see pv below)
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = 16 * G::slot(lane % 32, 2 * ks + hsel);
  const int tg = lane / 16;                            // 16-lane group
  const int tj = lane % 16;
  const int th = tg / 2;                               // key group of the B operand
  const int tdh = tg % 2;                              // which 16 d-columns
  int voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int R = 4 * th + tj / 4;
    const int dcol = 32 * db + 16 * tdh + 4 * (tj % 4);
    voff[db] = 16 * G::slot_v(R, dcol / 8) + 2 * (dcol % 8);
  }

  // ---- top of iteration t: wait for K(t) and V(t - 1)
  auto advance = [&](int t) { tile_barrier<G::OPS>(t); };
  // ---- the loads of iteration t (none in the last, PV-only one): issued
  //      inside the wave's VALU phase, which reads no LDS and leaves issue
  //      slots free while its exponentials run; one op before the first
  //      16-key chunk of exponentials and one after each of the next ones
  //      (ops [lo, hi) of a tensor per call). The early waves' VALU phase
  //      falls in the second half of an iteration, the late waves' in the
  //      first, so the two halves of the workgroup do not issue at once. Every
  //      op of iteration t still precedes the barrier of t + 1, in the order
  //      index slice, K(t + 3), V(t + 2): the wait counts hold.
  int knext[PW];
  auto issue_k = [&](int t, int lo = 0, int hi = kOpsEnd) {
    if (t < ti.ntiles) {
      if (lo == 0) {
        issue_index(t + IAHEAD);
        rows_from(t + KAHEAD, graw, knext);
      }
      issue_rows(kb, kring_lds, t + KAHEAD, knext, flag<false>{}, lo, hi);
    }
  };
  auto issue_v = [&](int t, int lo = 0, int hi = kOpsEnd) {
    if (t < ti.ntiles) {
      issue_rows(vb, vring_lds, t + VAHEAD, vrows, flag<true>{}, lo, hi);
      if (hi >= PW) {
#pragma unroll
        for (int i = 0; i < PW; ++i) vrows[i] = knext[i];
        read_gather(t + KAHEAD + 1, graw);               // used in the next iteration
      }
    }
  };
  // ---- the running max moved in the previous softmax: O to the new scale
  auto rescale = [&]() {
    if (resc) {
      // a real branch: without it the compiler multiplies O by a selected
      // factor (64 VALU ops) in every iteration
      asm volatile("");
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= corr;
      lacc *= corr;
      corr = 1.0f;
      resc = false;
    }
  };
  // ---- separator bits of band tile t (from its two rank slices); read in
  //      the MFMA phase, used by the VALU phase (the index slot may be
  //      reloaded before a late wave's VALU phase runs)
  auto sep_bits = [&](int t) -> uint64_t {
    if (t < ti.ntg) return 0;
    const int jmin = ti.band_lo + (t - ti.ntg) * KT;
    int r0 = idxr[t % IDXR][0][lane], r1 = idxr[t % IDXR][1][lane];
    asm volatile("" : "+v"(r0), "+v"(r1));            // read both unconditionally (no branch)
    return ballot((jmin + lane < Skv) & (r1 != r0));
  };
  // ---- V^T operand of PV MFMA i (16-key chunk kc = i / DB, d block
  //      db = i % DB) of the tile in V stage vst. O^T += V^T[:, chunk] . P^T:
  //      lane (16*tg + tj) points at key row 16*kc + 8*e + 4*th + tj/4, d
  //      column 32*db + 16*tdh + 4*(tj%4); the transpose load returns to
  //      lane l the keys {16*kc + 8*e + 4*th + k, k = 0..3} at d = 32*db + l%32.
  auto vread = [&](const char* vst, int i) -> bf16x8 {
    const int kc = i / DB, db = i % DB;
    const v4i16 x0 = read_tr16(vst + voff[db] + (16 * kc) * CPR * 16);
    const v4i16 x1 = read_tr16(vst + voff[db] + (16 * kc + 8) * CPR * 16);
    const v8i16 cat = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    return __builtin_bit_cast(bf16x8, cat);
  };
  constexpr int NMF = 4 * DB;                          // PV MFMAs per tile

  // ---- MFMA phase of iteration t: S^T of tile t into sh (two 32-key
  //      halves), then O^T += V^T P^T for tile t - 1 with pk
  auto mfma_phase = [&](int t, f32x16 (&sh)[2], auto do_qk, auto do_pv) {
    if constexpr (decltype(do_qk)::value) {
      const char* kst = kring + (t % KSTAGES) * TB;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(kst + koff[ks] + mb * 32 * CPR * 16));
          acc = mfma32x32x16(a, qf[ks], acc);
        }
        sh[mb] = acc;
      }
    }
    if constexpr (decltype(do_pv)::value) {
      const char* vst = vring + ((t + VSTAGES - 1) % VSTAGES) * TB;
#pragma unroll
      for (int i = 0; i < NMF; ++i)
        oacc[i % DB] = mfma32x32x16(vread(vst, i), __builtin_bit_cast(bf16x8, pk[i / DB]), oacc[i % DB]);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) lacc = mfma32x32x16(ones, __builtin_bit_cast(bf16x8, pk[kc]), lacc);
    }
    // a few LDS reads ahead of the MFMA that consumes them
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * KS + 2 * NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);                 // no VALU work mixed in
  };

  // ---- VALU phase for tile t: mask the scores where the tile needs it (a
  //      band tile whose keys all lie in the future of this wave's rows gets
  //      an all-zero visibility word, so its P is zero), then the online
  //      softmax into pk, m, l
  auto valu_phase = [&](int t, f32x16 (&sh)[2], uint64_t sepbits, int t_issue) {
    __builtin_amdgcn_sched_barrier(0);
    const bool band = t >= ti.ntg;
    const int jmin = band ? ti.band_lo + (t - ti.ntg) * KT : 0;
    const int nvalid = band ? KT : min(KT, ti.n_glob - t * KT);
    const bool full = band ? (jmin + KT - 1 <= qwv0 && jmin >= qmax - P.n + 1) : nvalid == KT;
    if (!full) {
      const uint64_t vis = vis_word(band, qi, jmin, P.n, P.a, sepbits, nvalid) >> (4 * hsel);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const uint32_t word = static_cast<uint32_t>(vis >> (32 * mb));
#pragma unroll
        for (int r = 0; r < 16; ++r) sh[mb][r] = mask_bit(sh[mb][r], word, 8 * (r / 4) + (r % 4));
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, sh[mb][r]);
    const float mx = half_max(m) * P.scale_log2;
    const bool grow = ballot(mx > m_run + kLazy) != 0ull;
    const float m_new = grow ? fmaxf(m_run, mx) : m_run;
    const float c = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
    corr *= c;
    m_run = m_new;
    resc = resc || grow;
    const float msub = (m_run == -INFINITY) ? 0.0f : m_run;
    issue_k(t_issue, 0, PW > 1 ? 1 : PW);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int o = 8 * (kc % 2);
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(__builtin_fmaf(sh[kc / 2][o + 2 * j], P.scale_log2, -msub));
        const float p1 = fast_exp2(__builtin_fmaf(sh[kc / 2][o + 2 * j + 1], P.scale_log2, -msub));
        w[j] = pack_bf16x2(p0, p1);
      }
      // computed here, in the VALU phase, not sunk into the MFMA phase
      // that consumes it
      asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
      pk[kc] = w;
      if (PW > 1 && kc == 0) issue_k(t_issue, 1, PW);
      if (PW > 1 && kc == 1) issue_v(t_issue, 0, 1);
      if (kc == 2) issue_v(t_issue, PW > 1 ? 1 : 0, PW);
    }
  };

  // The two waves that share a SIMD (waves w and w + 4) alternate between an
  // MFMA-only phase (QK of tile t and PV of tile t - 1) and a VALU-only phase
  // (mask and softmax), half an iteration apart, so that one wave's MFMAs
  // run while the other's VALU work does. Early waves: iteration t = MFMA(t),
  // VALU(t). Late waves: iteration t = VALU(t - 1), MFMA(t); their scores
  // wait in registers across the barrier. Both take ntiles + 1 barriers.
  f32x16 sh[2];
  uint64_t sepb = 0;
  if (wave < 4) {
    advance(0);
    mfma_phase(0, sh, flag<true>{}, flag<false>{});
    sepb = sep_bits(0);
    valu_phase(0, sh, sepb, 0);
    for (int t = 1; t < ti.ntiles; ++t) {
      advance(t);
      rescale();
      mfma_phase(t, sh, flag<true>{}, flag<true>{});
      sepb = sep_bits(t);
      valu_phase(t, sh, sepb, t);
    }
    advance(ti.ntiles);
    rescale();
    mfma_phase(ti.ntiles, sh, flag<false>{}, flag<true>{});
  } else {
    advance(0);
    mfma_phase(0, sh, flag<true>{}, flag<false>{});
    sepb = sep_bits(0);
    issue_k(0);                                        // (no VALU phase in iteration 0)
    issue_v(0);
    for (int t = 1; t < ti.ntiles; ++t) {
      advance(t);
      valu_phase(t - 1, sh, sepb, t);
      rescale();
      mfma_phase(t, sh, flag<true>{}, flag<true>{});
      sepb = sep_bits(t);
    }
    advance(ti.ntiles);
    valu_phase(ti.ntiles - 1, sh, sepb, ti.ntiles);
    rescale();
    mfma_phase(ti.ntiles, sh, flag<false>{}, flag<true>{});
  }

  // ---- epilogue: normalise, stage bf16 rows through LDS, store 16-byte chunks
  const float l_tot = lacc[0];
  const float inv = 1.0f / l_tot;
  // no LDS-DMA may still be landing in the ring (or after the wave ends)
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint16_t* stg = reinterpret_cast<uint16_t*>(ring) + wave * (32 * OSTR);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * hsel;
      u32x2 w;
      w[0] = pack_bf16x2(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv);
      w[1] = pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
      *reinterpret_cast<u32x2*>(stg + (lane % 32) * OSTR + d0) = w;
    }
  __syncthreads();
  uint16_t* ob = reinterpret_cast<uint16_t*>(P.out) + static_cast<int64_t>(b * P.Hq + h) * S * D;
  for (int e = lane; e < 32 * CPR; e += kWave) {
    const int r = e / CPR;
    const int c = e % CPR;
    const int row = qw0 + r;
    if (row < S)
      *reinterpret_cast<u32x4*>(ob + static_cast<int64_t>(row) * D + 8 * c) =
          *reinterpret_cast<const u32x4*>(stg + r * OSTR + 8 * c);
  }
  if (P.lse != nullptr && lane < 32 && qrow < S)
    P.lse[static_cast<int64_t>(b * P.Hq + h) * S + qrow] = (m_run + fast_log2(l_tot)) * kLn2;
}

}  // namespace

hipError_t launch_prefill_bf16(PrefillArgs A, int D, hipStream_t st) {
  A.QT = 32 * (NW / A.HPW);
  A.n_qt = (A.S + A.QT - 1) / A.QT;
  const int grid = A.B * A.Hkv * A.n_hg * A.n_qt;
  if (D == 128)
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3(grid), dim3(NT), 0, st, A);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3(grid), dim3(NT), 0, st, A);
  return hipGetLastError();
}

}  // namespace sep
