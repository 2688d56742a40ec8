// sep_attn_prefill, bf16 path: Sep-Attention prefill on 32x32x16 bf16 MFMA.
//
// Work decomposition (prefill.hpp): a workgroup owns one query tile of the
// HPW query heads that share a key/value head, and walks its key list
// (gathered initial + separator keys, then the dense band) in tiles of 64
// keys. Eight waves (two per SIMD) each hold 32 query rows of one head, so
// every K/V tile staged in LDS feeds 8 x 32 query rows.
//
// Staging: K and V tiles go straight from global memory into LDS with
// 16-byte LDS-DMA loads (no registers), into a ring of four stages, three
// tiles ahead of the tile being computed. Rows are stored row-major with
// the 16-byte chunk index XOR-swizzled by the row, one swizzle for K (the QK
// reads take one chunk of 32 rows) and one for V (a transposed read takes 64
// bytes of 4 rows per half wave), so that both hit distinct banks. The data
// a tile's gather needs (its slice of sep_pos, or for band tiles two
// shifted slices of rank whose difference gives the separator bits) also
// arrives by LDS-DMA, six tiles ahead, into an index ring. So the key loop
// has no global load with a register result: every wait is explicit. Each
// wave issues exactly OPS + 1 loads per iteration (a fixed dummy address
// past the last tile), waits with one exact vmcnt for its own loads of the
// current tile, and a plain barrier publishes them.
//
// Scores are computed transposed, S^T = K Q^T: each lane owns one query
// column, so a row max is a max over the lane's registers plus one exchange
// with lane l^32, and the exponentiated scores already sit in the B-operand
// layout of O^T = V^T P^T. The V^T A-operand is read with the LDS transpose
// load (ds_read_b64_tr_b16): pointing a 16-lane group at four consecutive key
// rows gives each lane four keys of one d column. Per tile, QK of the second
// 32-key half is issued before the softmax of the first half and PV of the
// first half before the softmax of the second. Softmax is online in fp32 in
// the log2 domain with lazy rescaling (the running max moves only when a
// row's max grows by more than 8), P is rounded to bf16 for the PV product.
#include "prefill.hpp"
#include "internal.hpp"

namespace sep {
namespace {

constexpr int KT = 64;                 // keys per tile
constexpr int NW = 8;                  // waves per workgroup
constexpr int NT = NW * kWave;
constexpr int STAGES = 4;              // LDS ring depth (tiles)
constexpr int AHEAD = STAGES - 1;      // tiles in flight ahead of the current one
constexpr int IAHEAD = 6;              // index slices loaded this many tiles ahead
constexpr int IDXR = 8;                // index ring depth (> IAHEAD)
constexpr float kLazy = 8.0f;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

template <int D>
struct Geo {
  static constexpr int CPR = D / 8;                    // 16-byte chunks per row
  static constexpr int TB = KT * D * 2;                // bytes of one K (or V) tile
  static constexpr int INSTR = TB / 1024;              // wave-wide 1 KB loads per tile
  static constexpr int PER_WAVE = INSTR / NW;          // per wave, per tensor
  static constexpr int OPS = 2 * PER_WAVE;             // LDS-DMA ops per wave per tile
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

// Wait until this wave's loads of tile t landed, then a plain barrier.
// Memory ops of a wave in issue order: the index slices of tiles 0..5 (one
// op each), [full wait], tiles 0, 1, 2 (OPS each); then per iteration one
// index-slice op followed by the OPS loads of tile t + 3. Ops issued after
// tile t's loads, at the top of iteration t: t = 0: 2*OPS; t = 1:
// 2*OPS + 1; t >= 2: 2*OPS + 2. Loads complete in issue order.
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

// Asynchronous global -> LDS copies. Lane l's 16 (or 4) bytes land at LDS
// address lds_base + 16*l (or + 4*l); lds_base is wave-uniform. There is no
// register result, so nothing waits for them except the explicit vmcnt.
// M0 carries the LDS base; the kernel makes no other use of M0 (no LDS-DMA
// builtins, no message or GWS instructions), so setting it inside the asm
// statement cannot disturb compiler-generated code.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_x4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void dma_x1(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(lds_base) : "memory", "m0");
}

#pragma clang diagnostic pop

__device__ __forceinline__ v4i16 read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
}

template <int D>
__global__ void __launch_bounds__(NT, 1) prefill_bf16_kernel(PrefillArgs P) {
  using G = Geo<D>;
  constexpr int CPR = G::CPR;
  constexpr int TB = G::TB;
  constexpr int KS = G::KS;
  constexpr int DB = G::DB;
  constexpr int OSTR = D + 8;                          // bf16 output-staging row stride
  static_assert(NW * 32 * OSTR * 2 <= STAGES * 2 * TB, "output staging must fit the ring");

  __shared__ __attribute__((aligned(1024))) char ring[STAGES * 2 * TB];
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
  const int S = P.S;
  const int q0 = qt * P.QT;
  const int q1 = min(q0 + P.QT, S);
  const int hw = wave % P.HPW;
  const int rb = wave / P.HPW;
  const int h = g * P.G + hg * P.HPW + hw;
  const int qw0 = q0 + 32 * rb;                        // this wave's first query row

  const int32_t* rk = P.rank + static_cast<int64_t>(b) * (S + 1);
  const int32_t* sp = P.sep_pos + static_cast<int64_t>(b) * S;
  const TileInfo ti = tile_info<KT>(rk, S, P.a, P.n, q0, q1);

  const uint16_t* kb = reinterpret_cast<const uint16_t*>(P.k) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(P.v) + static_cast<int64_t>(b * P.Hkv + g) * S * D;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(P.q) + static_cast<int64_t>(b * P.Hq + h) * S * D;

  // ---- index slice of tile t into ring slot t % IDXR: wave 0 loads
  //      sep_pos entries (global tiles) or rank[jmin + u]; wave 1 loads
  //      rank[jmin + u + 1] (band tiles); the other waves, and every wave
  //      past the last tile, load one fixed word into their junk row.
  auto issue_index = [&](int t) {
    const bool real = t < ti.ntiles;
    const bool band = t >= ti.ntg;
    const int32_t* src = rk;                           // fixed dummy address
    uint32_t dst = lds_addr(junk[wave]);
    if (real && wave < 2) {
      if (!band) {
        if (wave == 0) {
          const int si = min(max(ti.rank_a + t * KT + lane - ti.n_init, 0), S - 1);
          src = sp + si;
          dst = lds_addr(idxr[t % IDXR][0]);
        }
      } else {
        const int j = ti.band_lo + (t - ti.ntg) * KT + lane + wave;
        src = rk + min(j, S);
        dst = lds_addr(idxr[t % IDXR][wave]);
      }
    }
    dma_x1(src, __builtin_amdgcn_readfirstlane(dst));
  };
  // key row of entry r of tile t (from the index slice in LDS)
  auto key_of = [&](int t, int r) -> int {
    if (t >= ti.ntg) return min(ti.band_lo + (t - ti.ntg) * KT + r, S - 1);
    const int u = t * KT + r;
    if (u < ti.n_init) return u;
    if (u >= ti.n_glob) return 0;
    return idxr[t % IDXR][0][r];
  };
  // ---- LDS-DMA of tile t into ring stage t % STAGES. Past the last tile
  //      the same number of loads is issued (every lane re-reads one
  //      16-byte chunk into the unused stage).
  auto issue = [&](int t) {
    const bool real = t < ti.ntiles;
    char* kst = ring + (t % STAGES) * 2 * TB;
    char* vst = kst + TB;
#pragma unroll
    for (int i = 0; i < G::PER_WAVE; ++i) {
      const int ins = wave * G::PER_WAVE + i;          // 1 KB block of the tile
      const int sl = ins * kWave + lane;               // 16-byte slot this lane fills
      const int r = sl / CPR;
      const int pos = sl % CPR;
      const int64_t row = real ? static_cast<int64_t>(key_of(t, r)) * D : 0;
      const int64_t offk = real ? row + 8 * (pos ^ G::swz_k(r)) : 0;   // chunk that belongs in that slot
      const int64_t offv = real ? row + 8 * (pos ^ G::swz_v(r)) : 0;
      dma_x4(kb + offk, __builtin_amdgcn_readfirstlane(lds_addr(kst + ins * 1024)));
      dma_x4(vb + offv, __builtin_amdgcn_readfirstlane(lds_addr(vst + ins * 1024)));
    }
  };

  // ---- Q fragments first, so that waiting for them never waits for tiles
  bf16x8 qf[KS];
  {
    const int qrow = min(qw0 + lane % 32, S - 1);
    const uint16_t* p = qb + static_cast<int64_t>(qrow) * D + 8 * (lane / 32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p + 16 * ks));
  }
  for (int t = 0; t < IAHEAD; ++t) issue_index(t);
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0);                       // index slices 0..5 landed
  __syncthreads();
  for (int t = 0; t < AHEAD; ++t) issue(t);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const int qmax = min(qw0 + 31, S - 1);
  const int hsel = lane / 32;
  const int qi = qw0 + lane % 32;

  // per-lane pieces of the transposed V read address (see pv below)
  const int tg = lane / 16;                            // 16-lane group
  const int tj = lane % 16;
  const int th = tg / 2;                               // key group of the B operand
  const int tdh = tg % 2;                              // which 16 d-columns

  for (int t = 0; t < ti.ntiles; ++t) {
    tile_barrier<G::OPS>(t);
    issue_index(t + IAHEAD);
    issue(t + AHEAD);

    const char* kst = ring + (t % STAGES) * 2 * TB;
    const char* vst = kst + TB;
    const bool band = t >= ti.ntg;
    const int jmin = band ? ti.band_lo + (t - ti.ntg) * KT : 0;
    const int nvalid = band ? KT : min(KT, ti.n_glob - t * KT);
    bool skip = false, need_mask = false;
    if (band) {
      if (jmin > qmax || qw0 >= S) skip = true;        // every key in the future
      else need_mask = !(jmin + KT - 1 <= qw0 && jmin >= qmax - P.n + 1);
    } else {
      need_mask = nvalid < KT;
    }

    if (!skip) {
      uint64_t vis = 0;
      if (need_mask) {
        uint64_t sepbits = 0;
        if (band) {
          const int32_t* sl = idxr[t % IDXR][0];
          const bool f = (jmin + lane < S) && (idxr[t % IDXR][1][lane] != sl[lane]);
          sepbits = ballot(f);
        }
        vis = vis_word(band, qi, jmin, P.n, P.a, sepbits, nvalid) >> (4 * hsel);
      }
      // ---- S^T halves: keys 32*mb .. 32*mb+31 of the tile
      f32x16 sh[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 acc = {};
        const int r = 32 * mb + lane % 32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = 2 * ks + hsel;
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(kst + 16 * G::slot(r, c)));
          acc = mfma32x32x16(a, qf[ks], acc);
        }
        sh[mb] = acc;
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16& s = sh[mb];
        if (need_mask) {
          const uint32_t word = static_cast<uint32_t>(vis >> (32 * mb));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t bit = 1u << (8 * (r / 4) + (r % 4));
            s[r] = (word & bit) ? s[r] : -INFINITY;
          }
        }
        float m = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, s[r]);
        const float mx = fmaxf(m, swap_half(m)) * P.scale_log2;
        if (ballot(mx > m_run + kLazy) != 0ull) {
          const float m_new = fmaxf(m_run, mx);
          const float corr = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
          l_run *= corr;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] *= corr;
          m_run = m_new;
        }
        const float msub = (m_run == -INFINITY) ? 0.0f : m_run;
        float lsum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[r], P.scale_log2, -msub));
          s[r] = p;
          lsum += p;
        }
        l_run += lsum;
        // ---- O^T += V^T[:, keys of this half] . P^T
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int kc = 2 * mb + c2;                  // 16-key chunk of the tile
          u32x4 pk;
          pk[0] = pack_bf16x2(s[8 * c2 + 0], s[8 * c2 + 1]);
          pk[1] = pack_bf16x2(s[8 * c2 + 2], s[8 * c2 + 3]);
          pk[2] = pack_bf16x2(s[8 * c2 + 4], s[8 * c2 + 5]);
          pk[3] = pack_bf16x2(s[8 * c2 + 6], s[8 * c2 + 7]);
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            // lane (16*tg + tj) points at key row 16*kc + 8*e + 4*th + tj/4,
            // d column 32*db + 16*tdh + 4*(tj%4); the transpose load returns
            // to lane l the keys {16*kc + 8*e + 4*th + k, k = 0..3} at
            // d = 32*db + l%32.
            v4i16 x[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int R = 16 * kc + 8 * e + 4 * th + tj / 4;
              const int dcol = 32 * db + 16 * tdh + 4 * (tj % 4);
              x[e] = read_tr16(vst + 16 * G::slot_v(R, dcol / 8) + 2 * (dcol % 8));
            }
            const v8i16 cat = {x[0][0], x[0][1], x[0][2], x[0][3], x[1][0], x[1][1], x[1][2], x[1][3]};
            oacc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, cat), pb, oacc[db]);
          }
        }
      }
    }
  }

  // ---- epilogue: normalise, stage bf16 rows through LDS, store 16-byte chunks
  const float l_tot = l_run + swap_half(l_run);
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
  if (P.lse != nullptr && lane < 32 && qi < S)
    P.lse[static_cast<int64_t>(b * P.Hq + h) * S + qi] = (m_run + fast_log2(l_tot)) * kLn2;
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
