// Forward pass of fused exact attention for gfx950.
//
// Method: "FlashAttention core principles" (lesson 1), sections 3-4: the outer
// loop runs over query tiles (one workgroup per tile), the inner loop streams
// key/value tiles through on-chip memory, keeps a running row max m and row
// sum l, rescales the partial output by exp(m_old - m_new) when the max grows,
// and normalises once at the end. The single-exponential update of the
// interview answer ("2. Online Softmax") and of "FlashAttention and Triton",
// section 19.12 is used: p = exp(s - m), l = alpha*l + rowsum(p).
//
// gfx950 mapping
//   * Workgroup = 4 wave64s = BM = 128 query rows (32 per wave); two
//     workgroups per CU (8 waves), so two waves share each SIMD.
//   * Scores are computed transposed, S^T = K Q^T, with 32x32x16 bf16 MFMAs:
//     the accumulator holds one query per lane (column) and 16 keys per lane,
//     so row max / row sum are in-lane reductions plus one exchange between
//     the two 32-lane halves. O^T = V^T P^T keeps one query per lane as well:
//     P^T goes from the score accumulator into the B operand by register
//     conversion only, and the per-row rescale is a per-lane scalar.
//   * Q stays in registers for the whole key loop (B operand of S^T).
//   * K and V tiles go from HBM/L2 straight into LDS (global_load_lds_dwordx4,
//     no staging registers), row-major with XOR-swizzled 16-byte chunks so the
//     MFMA operand reads are free of bank conflicts. K operands are one
//     ds_read_b128 per lane; V^T operands come from the row-major V tile
//     through the transposing read ds_read_b64_tr_b16.
//   * K is prefetched two tiles ahead and V one tile ahead (two LDS buffers
//     each, one barrier per tile), and each wave is software-pipelined: the
//     S^T MFMAs of tile j+1 are issued next to the softmax VALU work of tile j
//     (one wave cannot overlap MFMA and VALU work unless its own instruction
//     stream interleaves them).
//   * Softmax runs in the base-2 domain with scale*log2(e) applied in fp32 (Q
//     is never pre-scaled in bf16); the running max moves only when a tile
//     max exceeds it by 2^8, which skips the O rescale on almost every tile
//     without changing the result (l and O share the reference max). LSE is
//     converted back to natural log on store.
//   * Causal: tiles above the diagonal are never loaded or computed; only
//     tiles crossing the diagonal (or the ragged end) evaluate the mask.
//     Query tiles are issued heaviest first, and the workgroups of one head
//     stay on one XCD (consecutive workgroup ids go to different XCDs).
//
// Long sequences at d = 128 use a second kernel, fa_fwd_pp_kernel (below):
// the same arithmetic in 256-row workgroups whose two 4-wave groups alternate
// MFMA and VALU clusters half a tile apart.
#include <type_traits>

#include "fa_common.h"

namespace fa {

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;               // query rows per workgroup
  static constexpr int THREADS = 256;          // 4 waves
  static constexpr int BN = 64;                // keys per tile
  static constexpr int RB = D * 2;             // bytes per K/V row in LDS
  static constexpr int TILE_BYTES = BN * RB;   // 16 KiB (d=128) or 8 KiB (d=64)
  static constexpr int LOADS = TILE_BYTES / 1024 / 4;   // 1 KiB DMAs per wave
  static constexpr int ROWS_PER_LOAD = 1024 / RB;
  static constexpr int NB = BN / 32;           // 32-key score blocks per tile
  static constexpr int DB = D / 32;            // 32-wide output blocks
  static constexpr int KS = D / 16;            // k-steps of S^T
  // One K or V tile copy follows each k-step of S^T (2*LOADS copies a step).
  static_assert(KS == 2 * LOADS, "one tile copy per k-step");
};

// Byte offset of (row, 16-byte chunk c) of a K tile in LDS. The XOR makes the
// 16 rows read by one MFMA operand load land in 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int k_off(int row, int c) {
  if constexpr (D == 128) return row * 256 + ((c ^ (row & 15)) << 4);
  else return row * 128 + ((c ^ ((row >> 1) & 7)) << 4);
}
// Byte offset of (row, column col) of a V tile in LDS: 64-byte blocks are
// XOR-swizzled so the 4 rows of one transposing read hit distinct banks.
template <int D>
__device__ __forceinline__ int v_off(int row, int col) {
  const int blk = col >> 5, in = (col & 31) * 2;
  if constexpr (D == 128) return row * 256 + ((blk ^ (row & 3)) << 6) + in;
  else return row * 128 + ((blk ^ ((row >> 1) & 1)) << 6) + in;
}

// Slack (log2 units) before the running max is moved.
constexpr float kRescaleSlack = 8.f;

// Max over the NB*16 score registers of a lane as a tree of 3-input maxima
// (v_maximum3_f32): 32 values in 16 instructions.
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }
template <int NB>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[NB]) {
  constexpr int n = NB * 16;
  float r[n];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) r[kb * 16 + i] = s[kb][i];
  int m = n;
#pragma unroll
  for (int level = 0; level < 6; ++level) {
    if (m == 1) break;
    int k = 0, i = 0;
#pragma unroll
    for (; i + 2 < m; i += 3) r[k++] = vmax3(r[i], r[i + 1], r[i + 2]);
    if (m - i == 2) r[k++] = vmax(r[i], r[i + 1]);
    else if (m - i == 1) r[k++] = r[i];
    m = k;
  }
  return r[0];
}
template <int NB>
__device__ __forceinline__ float tile_sum(const f32x16 (&s)[NB]) {
  float r[NB * 4];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      r[kb * 4 + g] = (s[kb][4 * g] + s[kb][4 * g + 1]) + (s[kb][4 * g + 2] + s[kb][4 * g + 3]);
#pragma unroll
  for (int w = NB * 4; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) r[i] = r[i] + r[i + w / 2];
  return r[0];
}

// Global -> LDS copies (global_load_lds_dwordx4: lane i writes LDS bytes
// [M0 + 16i, +16)), in the scalar-base form: the tile's base address is one
// SGPR pair and each lane adds a constant 32-bit byte offset, so a tile copy
// costs no per-lane address arithmetic. Issued from an asm statement (it
// writes M0, hence the clobber and the local pragma); the s_nop covers the
// M0-write -> LDS-DMA hazard. Completion is awaited with wait_dma() before
// the barrier that publishes a buffer.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
  strict_copy_wait();
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS void*)p;
}

// Byte offset (within a tile) of the global chunk that lane `lane` of this
// wave's copy i fetches: lane l writes physical 16-byte chunk l % (RB/16) of
// row lrow + l / (RB/16), so it reads the logical chunk the swizzle puts
// there. Rows are relative to the tile's first key.
template <int D, bool IS_V>
__device__ __forceinline__ int dma_row(int w, int i, int lane) {
  using C = FwdCfg<D>;
  return (w * C::LOADS + i) * C::ROWS_PER_LOAD + lane / (C::RB / 16);
}
template <int D, bool IS_V>
__device__ __forceinline__ int dma_col(int row, int lane) {
  using C = FwdCfg<D>;
  const int pc = lane % (C::RB / 16);                         // physical 16-byte chunk
  if constexpr (!IS_V) {
    int c;
    if constexpr (D == 128) c = pc ^ (row & 15);
    else c = pc ^ ((row >> 1) & 7);
    return c * 8;
  } else {
    const int pb = pc >> 2;
    int lb;
    if constexpr (D == 128) lb = pb ^ (row & 3);
    else lb = pb ^ ((row >> 1) & 1);
    return lb * 32 + (pc & 3) * 8;
  }
}

// This wave's share (LOADS x 1 KiB) of the copy of one K or V tile (keys
// kb0 .. kb0+BN-1). `off` holds the per-lane byte offsets for a full tile;
// on the ragged last tile, rows past N read row N-1 instead.
template <int D, bool IS_V>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, uint8_t* lds,
                                         int kb0, int N, int w, int lane,
                                         const uint32_t (&off)[FwdCfg<D>::LOADS]) {
  using C = FwdCfg<D>;
  const uint16_t* base = src + (size_t)kb0 * D;
  if (kb0 + C::BN <= N) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      lds_copy16(base, off[i], lds_addr_of(lds + (w * C::LOADS + i) * 1024));
  } else {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int row = dma_row<D, IS_V>(w, i, lane);
      const int r = min(row, N - 1 - kb0);
      const uint32_t o = (uint32_t)(r * D + dma_col<D, IS_V>(row, lane)) * 2u;
      lds_copy16(base, o, lds_addr_of(lds + (w * C::LOADS + i) * 1024));
    }
  }
}

// Copy i of this wave's share of a tile, branch-free: `full` / `ragged` are
// the per-lane offsets for a full tile and for the ragged last tile (the
// only tile that can be ragged).
template <int D>
__device__ __forceinline__ void dma_part(const uint16_t* __restrict__ src, uint8_t* lds,
                                         int kb0, int N, int w, int i, uint32_t full,
                                         uint32_t ragged) {
  using C = FwdCfg<D>;
  const uint32_t o = (kb0 + C::BN <= N) ? full : ragged;
  lds_copy16(src + (size_t)kb0 * D, o, lds_addr_of(lds + (w * C::LOADS + i) * 1024));
}

__device__ __forceinline__ void wait_dma() {
  // s_waitcnt vmcnt(0): this wave's outstanding global->LDS copies are done.
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// POS: scale > 0. Then a masked score can be stored as a raw -inf (its
// scaled value is -inf as well) and every tile uses exp2(fma(s, c2, -m)).
// Otherwise (scale <= 0, rare) every tile is scaled first and uses
// exp2(s - m).
// Item b (a workgroup, or an item of the persistent kernel) -> (head, query
// tile rank; rank 0 = heaviest causal tile).
__device__ __forceinline__ void item_to_tile(int b, int BH, int xcd_group, int& head, int& rank,
                                             int ntq = 0, bool complement = false) {
  if (xcd_group > 0) {
    // Workgroups are dispatched round-robin over the 8 XCDs; give XCD x the
    // heads [x*G, (x+1)*G) so their K/V stay in that XCD's L2.
    const int x = b & 7, s = b >> 3;
    // Item i of the XCD's heaviest-first list (heads interleaved per rank).
    // complement: a one-round grid whose workgroups the dispatcher places
    // breadth-first, slot 0 of the XCD's 32 CUs for s = 0..31, then slot 1
    // for s = 32..; the second pass takes the list from its light end, so
    // the CU holding the i-th heaviest tile also holds the i-th lightest.
    const int i = (complement && s >= 32) ? ntq * xcd_group + 31 - s : s;
    head = x * xcd_group + i % xcd_group;
    rank = i / xcd_group;
  } else {
    head = b % BH;
    rank = b / BH;
  }
}

// One 128-row query tile (`rank`-th heaviest of head `head`): the whole
// online-softmax pass and its epilogue, on the four LDS buffers given (each
// G * TILE_BYTES bytes). Called once per workgroup by fa_fwd_kernel and once
// per item by the persistent comparator kernel.
template <int D, bool CAUSAL, bool POS, int G>
__device__ __forceinline__ void fwd_tile(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int N, int ntq, float c2, int head, int rank, int tid,
    uint8_t* k_lds0, uint8_t* k_lds1, uint8_t* v_lds0, uint8_t* v_lds1) {
  using C = FwdCfg<D>;
  const int lane = tid & 63;
  const int wall = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  // G = 2: two groups of 4 waves own the same 128 rows; group g takes the key
  // tiles g, g+2, g+4, ... into its own half of each LDS buffer. Waves i and
  // i+4 share a SIMD.
  const int w = G == 1 ? wall : (wall & 3);
  const int grp = G == 1 ? 0 : (wall >> 2);
  const int gofs = grp * C::TILE_BYTES;   // this group's half of each buffer
  const int l32 = lane & 31, hi = lane >> 5;

  const int qt = CAUSAL ? (ntq - 1 - rank) : rank;
  const int q0 = qt * C::BM;
  const int qw = q0 + w * 32;          // first query row of this wave
  const int qrow = qw + l32;           // this lane's query row
  const size_t off = (size_t)head * N * D;
  const uint16_t* Kh = K + off;
  const uint16_t* Vh = V + off;

  const int kend = CAUSAL ? min(N, q0 + C::BM) : N;
  const int nt = (kend + C::BN - 1) / C::BN;
  // Key tiles this wave computes: 0 .. ntw-1 (causal waves stop at the diagonal).
  const int ntw = CAUSAL ? min(nt, (min(N, qw + 32) + C::BN - 1) / C::BN) : nt;
  // Its group's share: local tile i is key tile G*i + grp; ns steps for all.
  const int ns = (nt + G - 1) / G;
  const int ntw_g = (ntw - grp + G - 1) / G;
  auto kbase_of = [&](int i) { return min(G * i + grp, nt - 1) * C::BN; };

  // Per-lane byte offsets of the K and V tile copies (constant across tiles).
  uint32_t koffd[C::LOADS], voffd[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int rk = dma_row<D, false>(w, i, lane);
    koffd[i] = (uint32_t)(rk * D + dma_col<D, false>(rk, lane)) * 2u;
    const int rv = dma_row<D, true>(w, i, lane);
    voffd[i] = (uint32_t)(rv * D + dma_col<D, true>(rv, lane)) * 2u;
  }
  // The same for the last tile when it is ragged (rows past N read row N-1).
  uint32_t koffr[C::LOADS], voffr[C::LOADS];
  {
    const int kl = (nt - 1) * C::BN;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int rk = dma_row<D, false>(w, i, lane);
      koffr[i] = (uint32_t)(min(rk, N - 1 - kl) * D + dma_col<D, false>(rk, lane)) * 2u;
      const int rv = dma_row<D, true>(w, i, lane);
      voffr[i] = (uint32_t)(min(rv, N - 1 - kl) * D + dma_col<D, true>(rv, lane)) * 2u;
    }
  }

  // Prologue DMA: K0, V0, K1 (of this group's tiles).
  dma_tile<D, false>(Kh, k_lds0 + gofs, kbase_of(0), N, w, lane, koffd);
  dma_tile<D, true>(Vh, v_lds0 + gofs, kbase_of(0), N, w, lane, voffd);
  if (ns > 1) dma_tile<D, false>(Kh, k_lds1 + gofs, kbase_of(1), N, w, lane, koffd);

  // Q rows of this lane as B operands (rows past N read row N-1; never stored).
  bf16x8 qreg[C::KS];
  {
    const uint16_t* qp = Q + off + (size_t)min(qrow, N - 1) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qreg[ks] = __builtin_bit_cast(bf16x8, ld_global_16B(qp + ks * 16));
  }

  // Per-lane LDS read offsets. K operand (row kb*32 + l32, chunk 2ks + hi):
  // the row's swizzle only depends on l32, so the 32-row block kb is an
  // immediate offset and one register per k-step holds the XORed chunk.
  int koff[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) koff[ks] = k_off<D>(l32, 2 * ks + hi) + gofs;
  // Transposing V reads: lane (group g = lane/16, source s = lane%16) points
  // at V row 16t + 8*half + 4*hi + s/4, columns 32*db + 16*(g&1) + 4*(s&3)..+3.
  // The swizzle of those rows only depends on s, so t and the half are
  // immediate offsets and one register per 32-column block db remains.
  int voff[C::DB];
  {
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      voff[db] = v_off<D>(4 * hi + (sl >> 2), 32 * db + 16 * (g & 1) + 4 * (sl & 3)) + gofs;
  }

  f32x16 oacc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;   // running (reference) max of this lane's row, log2 domain
  float l_run = 0.f;         // running sum over this lane's half of the keys

  auto scores = [&](f32x16 (&s)[C::NB], const uint8_t* kt, auto&& hook) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < C::NB; ++kb) s[kb] = zero16();
    // k-step outer: consecutive MFMAs alternate between the independent
    // accumulators of the 32-key blocks instead of waiting on one chain.
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < C::NB; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + kb * 32 * C::RB + koff[ks]);
        s[kb] = mfma_32x32x16(a, qreg[ks], s[kb]);
      }
      hook(ks);
    }
  };

  f32x16 sacc[2][C::NB];   // scores of tiles j (parity of j) and j+1

  // Statistics of a freshly computed score tile: mask it if it crosses the
  // diagonal or the ragged end (masked tiles are left scaled by c2, others
  // raw), take its max, exchange it between the two row halves, and move
  // the reference max if it grew by more than kRescaleSlack (rare: O and l
  // are rescaled then). Returns whether the tile was masked.
  auto tile_stats = [&](f32x16 (&s)[C::NB], int kbase) __attribute__((always_inline)) {
    const bool masked = (CAUSAL && kbase + C::BN - 1 > qw) || (kbase + C::BN > N);
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
          const bool ok = key < N && (!CAUSAL || key <= qrow);
          if constexpr (POS) s[kb][i] = ok ? s[kb][i] : -INFINITY;
          else s[kb][i] = ok ? s[kb][i] * c2 : -INFINITY;
        }
    } else if constexpr (!POS) {
#pragma unroll
      for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] *= c2;
    }
    float tmax = tile_max<C::NB>(s);
    if constexpr (POS) tmax *= c2;
    tmax = halves_max(tmax);
    const bool grow = tmax > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? tmax : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
  };

  // The branch-free body of a tile step: S^T of the next tile (MFMA, when
  // HAS_NEXT) beside p = exp2(s - m), the row sum, the bf16 packing and
  // O^T += V^T P^T of this tile, so the scheduler can interleave MFMA and
  // VALU work of one wave.
  auto tile_body = [&](f32x16 (&scur)[C::NB], f32x16 (&snext)[C::NB], const uint8_t* k_next,
                       const uint8_t* v_this, auto&& copy) __attribute__((always_inline)) {
    scores(snext, k_next, copy);
    // A row with no admissible key so far keeps m = -inf (all its scores
    // are -inf): subtract 0 so that p = 0.
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    if constexpr (!POS) {
#pragma unroll
      for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) scur[kb][i] = fast_exp2(scur[kb][i] - m_use);
    } else {
      const float nm = -m_use;
#pragma unroll
      for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) scur[kb][i] = fast_exp2(fmaf(scur[kb][i], c2, nm));
    }
    // O^T += V^T P^T: 16 keys per MFMA; k-slot s of half h is key
    // 8*(s/4) + 4h + s%4 of the 16, both in P^T (accumulator rows) and in
    // the V^T operand (two transposing reads of 4 keys each).
#pragma unroll
    for (int t = 0; t < C::BN / 16; ++t) {
      const f32x16& p = scur[t >> 1];
      const int r0 = (t & 1) * 8;
      const bf16x8 pb = pack_bf16x8(p[r0 + 0], p[r0 + 1], p[r0 + 2], p[r0 + 3],
                                    p[r0 + 4], p[r0 + 5], p[r0 + 6], p[r0 + 7]);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const uint8_t* vp = v_this + 16 * t * C::RB + voff[db];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)vp);
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vp + 8 * C::RB));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = mfma_32x32x16(a, pb, oacc[db]);
      }
    }
    // The row sum is taken over the fp32 p (a sum of the bf16-rounded p would
    // move the LSE by up to 2^-9 on rows with few keys).
    l_run += tile_sum<C::NB>(scur);
    // Instruction order for this block (one wave issues in order, so MFMA
    // work only overlaps VALU work that sits between the MFMAs, and LDS
    // latency is only hidden by reads issued several MFMAs ahead): the S^T
    // MFMAs of the next tile each carry two LDS reads (the remaining K
    // operands, then the first V^T operands of the O^T phase) and the
    // fma+exp of two scores; the O^T MFMAs each carry one V^T read and the
    // row-sum / bf16-pack work.
    constexpr int kMfma = 0x008, kValu = 0x002, kDsRead = 0x100;
    __builtin_amdgcn_sched_group_barrier(kDsRead, 4, 0);
#pragma unroll
    for (int i = 0; i < C::NB * C::KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kValu, 4, 0);
    }
#pragma unroll
    for (int i = 0; i < (C::BN / 16) * C::DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kValu, 3, 0);
    }
  };

  wait_dma();
  __syncthreads();
  if (ntw_g > 0) {
    scores(sacc[0], k_lds0, [](int) {});
    tile_stats(sacc[0], grp * C::BN);
  }
  __syncthreads();   // K buffer 0 is refilled by the first tile step

  // One tile step; P is the parity of j (K_j and V_j live in buffer P).
  // Entering it, sacc[P] holds tile j's scores (masked, and with the
  // reference max already updated for them).
  auto step = [&](auto parity, int j) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    uint8_t* const k_this = P ? k_lds1 : k_lds0;   // K_j (done), refilled with K_{j+2}
    uint8_t* const k_next = P ? k_lds0 : k_lds1;   // K_{j+1}
    uint8_t* const v_this = P ? v_lds1 : v_lds0;   // V_j
    uint8_t* const v_next = P ? v_lds0 : v_lds1;   // refilled with V_{j+1}
    // Copies of K_{j+2} and V_{j+1} (copy c: K part c/2 for even c, V part
    // c/2 for odd c), one after each k-step of the S^T MFMAs: spread out so
    // they do not stall instruction issue as a burst would, and all in the
    // first half of the step so they complete before the closing barrier.
    // Near the end they repeat the last tile (in bounds, unused).
    const int kc0 = kbase_of(j + 2), vc0 = kbase_of(j + 1);
    auto copy = [&](int c) __attribute__((always_inline)) {
      const int i = c >> 1;
      if (c & 1) dma_part<D>(Vh, v_next + gofs, vc0, N, w, i, voffd[i], voffr[i]);
      else dma_part<D>(Kh, k_this + gofs, kc0, N, w, i, koffd[i], koffr[i]);
    };
    f32x16 (&scur)[C::NB] = sacc[P];
    f32x16 (&snext)[C::NB] = sacc[P ^ 1];
    if (j < ntw_g) {
      // The next tile's scores are computed even on this wave's last tile
      // (then from whatever the other K buffer holds, and never used): one
      // code path keeps the register allocation of the loop simple.
      tile_body(scur, snext, k_next, v_this, copy);
      if (j + 1 < ntw_g) tile_stats(snext, (G * (j + 1) + grp) * C::BN);
    } else {
#pragma unroll
      for (int c = 0; c < 2 * C::LOADS; ++c) copy(c);
    }
    wait_dma();
    __syncthreads();
  };

  for (int j = 0; j < ns; j += 2) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ns) step(std::integral_constant<int, 1>{}, j + 1);
  }

  if constexpr (G == 2) {
    // Group 1 hands its reference max, its row-half sums and its O^T partials
    // to the group-0 wave with the same rows and lanes (through its own, now
    // idle, LDS halves), which rescales both to the larger max and adds them.
    float* const xo = reinterpret_cast<float*>(
        (w == 0 ? k_lds0 : w == 1 ? k_lds1 : w == 2 ? v_lds0 : v_lds1) + C::TILE_BYTES);
    float* const xs = reinterpret_cast<float*>(v_lds1) + w * 128;
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(xo + ((db * 4 + q4) * 64 + lane) * 4) =
              f32x4{oacc[db][4 * q4], oacc[db][4 * q4 + 1], oacc[db][4 * q4 + 2], oacc[db][4 * q4 + 3]};
      xs[lane] = m_run;
      xs[64 + lane] = l_run;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xs[lane], l1 = xs[64 + lane];
    const float m = vmax(m_run, m1);
    const float mu = m == -INFINITY ? 0.f : m;
    const float a0 = fast_exp2(m_run - mu), a1 = fast_exp2(m1 - mu);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 p = *reinterpret_cast<const f32x4*>(xo + ((db * 4 + q4) * 64 + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[db][4 * q4 + e] = fmaf(p[e], a1, oacc[db][4 * q4 + e] * a0);
      }
    l_run = fmaf(l1, a1, l_run * a0);
    m_run = m;
  }

  // ---- epilogue: O = O / l, LSE = ln2 * (m + log2 l). O leaves through
  // this wave's slice of the K buffers (free: every step ended with a
  // barrier after its reads and copies).
  const float l_tot = halves_sum(l_run);
  {
    const float inv = 1.f / l_tot;
    u32x2 ov[C::DB][4];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        ov[db][g4] = u32x2{pack_bf16x2(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv),
                           pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
    store_rows_staged<D>(O + off + (size_t)qw * D, N - qw, (w < 2 ? k_lds0 : k_lds1) + (w & 1) * 32 * C::RB,
                         ov, lane);
  }
  if (qrow < N && hi == 0) LSE[(size_t)head * N + qrow] = (m_run + fast_log2(l_tot)) * kLn2;
}

template <int D, bool CAUSAL, bool POS, int G>
__global__ __launch_bounds__(256 * G) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int BH, int N, int ntq, float c2, int xcd_group, int complement) {
  using C = FwdCfg<D>;
  // Four distinct LDS objects (not one indexed array): the loop below is
  // unrolled by two so each access names its buffer statically, which lets
  // the compiler see that an in-flight DMA into one buffer does not alias
  // the reads of another (otherwise it waits for the DMA before every read).
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[G * C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[G * C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[G * C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[G * C::TILE_BYTES];

  // Workgroup -> (head, query tile).
  int head, rank;
  item_to_tile(blockIdx.x, BH, xcd_group, head, rank, ntq, complement != 0);
  fwd_tile<D, CAUSAL, POS, G>(Q, K, V, O, LSE, N, ntq, c2, head, rank, threadIdx.x, k_lds0,
                              k_lds1, v_lds0, v_lds1);
}

// Comparator: the same forward pass on a persistent grid. At most two 4-wave
// workgroups per CU (512) stay resident and each loops over query tiles
// ("items", the workgroups of fa_fwd_kernel in its heaviest-first order).
// The schedule is static: within the items of each XCD, round k gives
// workgroup g the k-th block of items in "snake" order (g in even rounds,
// the mirror position in odd ones), so a workgroup that draws a heavy
// causal tile in one round draws a light one in the next. fa_fwd_kernel
// instead leaves the balancing to the hardware dispatcher, which starts each
// next workgroup on whichever slot frees first. The loop state (round, item)
// is uniform and lives in scalar registers.
template <int D, bool CAUSAL, bool POS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_persistent_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int BH, int N, int ntq, float c2, int xcd_group) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[C::TILE_BYTES];
  const int total = ntq * BH;
  // Items of one XCD (b = 8s + x) when the heads are grouped by XCD, else
  // all items (b = s); P workgroups share them, PL per XCD.
  const int groups = xcd_group > 0 ? 8 : 1;
  const int g = blockIdx.x;
  const int x = g % groups, gl = g / groups;
  const int PL = gridDim.x / groups, TL = total / groups;
  for (int k = 0;; ++k) {
    const int s = k * PL + ((k & 1) ? PL - 1 - gl : gl);
    if (s >= TL) break;   // s grows with k for every workgroup
    if (k > 0) __syncthreads();   // the previous item's LDS reads and stores are done
    int head, rank;
    item_to_tile(s * groups + x, BH, xcd_group, head, rank);
    // The thread id, the pointers and the sizes pass through empty asm
    // statements: everything derived from them is then recomputed per item
    // rather than hoisted out of the loop and held in registers across it.
    int tid = threadIdx.x, n = N, nq = ntq;
    float c = c2;
    const uint16_t *q = Q, *kk = K, *vv = V;
    uint16_t* o = O;
    float* lse = LSE;
    asm volatile("" : "+v"(tid));
    asm volatile("" : "+s"(n), "+s"(nq), "+s"(c), "+s"(q), "+s"(kk), "+s"(vv), "+s"(o), "+s"(lse));
    fwd_tile<D, CAUSAL, POS, 1>(q, kk, vv, o, lse, n, nq, c, head, rank, tid, k_lds0, k_lds1,
                                v_lds0, v_lds1);
  }
}

template <int D, bool CAUSAL, bool POS>
static hipError_t launch_fwd_persistent(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        uint16_t* o, float* lse, int BH, int N, float scale,
                                        hipStream_t stream) {
  using C = FwdCfg<D>;
  const int ntq = (N + C::BM - 1) / C::BM;
  const int xcd_group = (BH % 8 == 0) ? BH / 8 : 0;
  const float c2 = scale * kLog2e;
  // Two resident workgroups per CU on 256 CUs (a multiple of 8, so that
  // workgroup g runs on XCD g % 8), or one per item if there are fewer.
  const int total = ntq * BH;
  const int nwg = total < 512 ? total : 512;
  hipLaunchKernelGGL((fa_fwd_persistent_kernel<D, CAUSAL, POS>), dim3((unsigned)nwg),
                     dim3(C::THREADS), 0, stream, q, k, v, o, lse, BH, N, ntq, c2, xcd_group);
  return hipGetLastError();
}

hipError_t fwd_persistent_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* o, float* lse, int BH, int N, int d, float scale,
                                   bool causal, hipStream_t stream) {
  const bool pos = scale > 0.f;
#define FA_FWDP_CASE(DD, CC, PP) \
  if (d == DD && causal == CC && pos == PP) \
    return launch_fwd_persistent<DD, CC, PP>(q, k, v, o, lse, BH, N, scale, stream);
  FA_FWDP_CASE(128, true, true)
  FA_FWDP_CASE(128, false, true)
  FA_FWDP_CASE(64, true, true)
  FA_FWDP_CASE(64, false, true)
  FA_FWDP_CASE(128, true, false)
  FA_FWDP_CASE(128, false, false)
  FA_FWDP_CASE(64, true, false)
  FA_FWDP_CASE(64, false, false)
#undef FA_FWDP_CASE
  return hipErrorInvalidValue;
}

// d = 64 grids of at most 256 128-row query tiles (one per CU) with at least
// 1024 keys: 8-wave workgroups whose two 4-wave groups split the key tiles of
// the same 128 rows (G = 2 above). Measured 16-20 % faster (B=1: H=8, N=4096
// causal and not; H=4, N=8192 causal; H=16, N=2048 causal), where one 4-wave
// workgroup per CU leaves one wave per SIMD. Where two workgroups share each
// CU, independent workgroups run out of phase and the lockstep groups lose
// (+7.7 % at B=2, H=16, N=2048, d=128).
bool fwd_uses_split_groups(int BH, int N, int d) {
  return d == 64 && N >= 1024 && (long)((N + 127) / 128) * BH <= 256;
}

template <int D, bool CAUSAL, bool POS>
static hipError_t launch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint16_t* o, float* lse, int BH, int N, float scale,
                             hipStream_t stream) {
  using C = FwdCfg<D>;
  const int ntq = (N + C::BM - 1) / C::BM;
  const int xcd_group = (BH % 8 == 0) ? BH / 8 : 0;
  const float c2 = scale * kLog2e;
  dim3 grid((unsigned)(ntq * BH));
  if (fwd_uses_split_groups(BH, N, D)) {
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, POS, 2>), grid, dim3(2 * C::THREADS), 0, stream,
                       q, k, v, o, lse, BH, N, ntq, c2, xcd_group, 0);
  } else {
    // Causal grids of one round (257-512 tiles, two workgroups per CU):
    // heavy and light tiles share each CU.
    const int complement = CAUSAL && xcd_group > 0 && ntq * BH > 256 && ntq * BH <= 512;
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, POS, 1>), grid, dim3(C::THREADS), 0, stream,
                       q, k, v, o, lse, BH, N, ntq, c2, xcd_group, complement);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// d = 128 forward, 256 query rows per workgroup in two groups of 4 waves that
// alternate MFMA and VALU work ("ping-pong").
//
// Each wave owns 32 query rows and runs the same online-softmax recurrence as
// fa_fwd_kernel, but cut into two clusters per key tile j:
//   M(j): S^T of tile j+1 (16 MFMAs) and O^T += V_j^T P_j^T (16 MFMAs) -- MFMA
//         and LDS operand reads only;
//   V(j): the statistics of tile j+1 (mask, max, reference-max update),
//         P_{j+1} = exp2(s - m), its row sum and bf16 packing, and this
//         group's tile copies -- VALU and copies only.
// Group 1 runs half a tile behind group 0 and every cluster ends at a
// workgroup barrier, so while one wave of a SIMD is in its MFMA cluster the
// other (waves i and i+4 share a SIMD) is in its VALU cluster. K and V tiles
// of 64 keys are double-buffered in LDS (64 KiB, so every operand read keeps
// an immediate offset); group 1 issues every tile copy, in its VALU
// clusters, and waits for it at the end of its next MFMA cluster.
//
// SPLIT (grids of at most one 128-row tile per CU): both groups own the same
// 128 query rows and split the key tiles between them, group g taking tiles
// g, g+2, g+4, ... into its own half of each buffer (128 KiB) and copying
// them itself. Each group's softmax statistics and O are partial; at the end
// group 1 passes its max, row sums and O accumulators through LDS and group 0
// rescales both parts to the larger max (exp2 of the differences), adds them
// and stores. On such grids the one-group kernel leaves one wave per SIMD
// with nothing to overlap with; here two waves of each SIMD alternate MFMA
// and VALU clusters, and the longest row's key tiles are shared by two waves.
//
// PAIR (causal SPLIT grids of up to two 128-row tiles per CU): each
// workgroup runs two query tiles one after the other, the heavy tile
// ntq-1-u and the light tile u, so all workgroups have the same number of
// key tiles and the grid fits in one round.
// ---------------------------------------------------------------------------
struct PingPongCfg {
  static constexpr int D = 128, BM = 256, THREADS = 512, BN = 64, RB = 256;
  static constexpr int TILE = BN * RB;           // 16 KiB
  static constexpr int LOADS = TILE / 1024 / 4;  // 1 KiB copies per wave of a group (4)
  static constexpr int NB = 2, DB = 4, KS = 8;
};


template <bool CAUSAL, bool POS, bool SPLIT, bool PAIR = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_pp_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int BH, int N, int ntq, float c2, int xcd_group) {
  using C = PingPongCfg;
  using FC = FwdCfg<128>;
  constexpr int D = C::D, RB = C::RB, BN = C::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t kl0[(SPLIT ? 2 : 1) * C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kl1[(SPLIT ? 2 : 1) * C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vl0[(SPLIT ? 2 : 1) * C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vl1[(SPLIT ? 2 : 1) * C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wall = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wall >> 2;            // 0: waves 0-3, 1: waves 4-7 (wave i and i+4 share a SIMD)
  const int w = wall & 3;               // wave within the group
  // SPLIT: both groups own the same 128 rows (block w) and take alternate key
  // tiles (group g: local tile j is key tile 2j + g), each in its own half of
  // every LDS buffer; the two partial results are merged at the end.
  const int blk = SPLIT ? w : 2 * w + grp;   // this wave's 32-row block
  constexpr int BMQ = SPLIT ? 128 : C::BM;   // query rows per workgroup
  const int gofs = SPLIT ? grp * C::TILE : 0;
  const int l32 = lane & 31, hi = lane >> 5;

  int head, rank;
  {
    const int b = blockIdx.x;
    if (xcd_group > 0) {
      const int x = b & 7, s = b >> 3;
      head = x * xcd_group + s % xcd_group;
      rank = s / xcd_group;
    } else {
      head = b % BH;
      rank = b / BH;
    }
  }
  static_assert(!PAIR || (SPLIT && CAUSAL), "pairs are causal split-key tiles");
  // One query tile `qt` (128 rows with SPLIT, else 256).
  auto item = [&](const int qt) __attribute__((always_inline)) {
    const int q0 = qt * BMQ;
    const int qw = q0 + 32 * blk;
    const int qrow = qw + l32;
    const size_t off = (size_t)head * N * D;
    const uint16_t* Kh = K + off;
    const uint16_t* Vh = V + off;

    const int kend = CAUSAL ? min(N, q0 + BMQ) : N;
    const int nt = (kend + BN - 1) / BN;
    const int ntw_all = CAUSAL ? min(nt, (min(N, qw + 32) + BN - 1) / BN) : nt;
    // Steps (the same for every wave) and this wave's computed local tiles.
    const int ns = SPLIT ? (nt + 1) >> 1 : nt;
    const int ntw = SPLIT ? (ntw_all - grp + 1) >> 1 : ntw_all;
    auto key_tile = [&](int j) { return SPLIT ? 2 * j + grp : j; };

    static_assert(FC::LOADS == C::LOADS, "copy layout shared with fa_fwd_kernel");
    // This group's 4 waves copy tile t (tiles past the last repeat it: in
    // bounds, unused) of K (IS_V false) or V into dst, in the layout of
    // fa_fwd_kernel's copies (rows past N read row N-1). The per-lane offsets
    // are formed here, in the VALU cluster, rather than held in registers.
    auto copy_tile = [&](auto is_v, uint8_t* dst, int t) __attribute__((always_inline)) {
      constexpr bool IS_V = decltype(is_v)::value;
      const int kb0 = min(key_tile(t), nt - 1) * BN;
      const int rmax = N - 1 - kb0;
  #pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        const int r = dma_row<128, IS_V>(w, i, lane);
        const uint32_t o = (uint32_t)(min(r, rmax) * D + dma_col<128, IS_V>(r, lane)) * 2u;
        lds_copy16((IS_V ? Vh : Kh) + (size_t)kb0 * D, o,
                   lds_addr_of(dst + gofs + (w * C::LOADS + i) * 1024));
      }
    };
    using KT = std::integral_constant<bool, false>;
    using VT = std::integral_constant<bool, true>;

    bf16x8 qreg[C::KS];
    {
      const uint16_t* qp = Q + off + (size_t)min(qrow, N - 1) * D + hi * 8;
  #pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        qreg[ks] = __builtin_bit_cast(bf16x8, ld_global_16B(qp + ks * 16));
    }
    // Prologue copies: K_0 and K_1 (group 0), V_0 and V_1 (group 1); with
    // SPLIT every group copies its own four.
    if (SPLIT) {
      copy_tile(KT{}, kl0, 0);
      copy_tile(KT{}, kl1, 1);
      copy_tile(VT{}, vl0, 0);
      copy_tile(VT{}, vl1, 1);
    } else if (grp == 0) {
      copy_tile(KT{}, kl0, 0);
      copy_tile(KT{}, kl1, 1);
    } else {
      copy_tile(VT{}, vl0, 0);
      copy_tile(VT{}, vl1, 1);
    }

    int koff[C::KS];
  #pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) koff[ks] = k_off<D>(l32, 2 * ks + hi) + gofs;
    int voff[C::DB];
    {
      const int g = lane >> 4, sl = lane & 15;
  #pragma unroll
      for (int db = 0; db < C::DB; ++db)
        voff[db] = v_off<D>(4 * hi + (sl >> 2), 32 * db + 16 * (g & 1) + 4 * (sl & 3)) + gofs;
    }

    f32x16 oacc[C::DB];
  #pragma unroll
    for (int i = 0; i < C::DB; ++i) oacc[i] = zero16();
    f32x16 sacc[C::NB];
    bf16x8 pk[BN / 16];
    float m_run = -INFINITY, l_run = 0.f;

    auto scores = [&](const uint8_t* kt) __attribute__((always_inline)) {
  #pragma unroll
      for (int kb = 0; kb < C::NB; ++kb) sacc[kb] = zero16();
  #pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
  #pragma unroll
        for (int kb = 0; kb < C::NB; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + kb * 32 * RB + koff[ks]);
          sacc[kb] = mfma_32x32x16(a, qreg[ks], sacc[kb]);
        }
    };
    auto pv = [&](const uint8_t* vt) __attribute__((always_inline)) {
  #pragma unroll
      for (int t = 0; t < BN / 16; ++t)
  #pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const uint8_t* vp = vt + 16 * t * RB + voff[db];
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)vp);
          const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vp + 8 * RB));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = mfma_32x32x16(a, pk[t], oacc[db]);
        }
    };
    // Statistics of tile kbase (as in fa_fwd_kernel), then P = exp2(s - m) for
    // it, its row sum and bf16 packing into the next PV operands.
    auto softmax = [&](int kbase) __attribute__((always_inline)) {
      const bool masked = (CAUSAL && kbase + BN - 1 > qw) || (kbase + BN > N);
      if (masked) {
  #pragma unroll
        for (int kb = 0; kb < C::NB; ++kb)
  #pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kbase + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
            const bool ok = key < N && (!CAUSAL || key <= qrow);
            if constexpr (POS) sacc[kb][i] = ok ? sacc[kb][i] : -INFINITY;
            else sacc[kb][i] = ok ? sacc[kb][i] * c2 : -INFINITY;
          }
      } else if constexpr (!POS) {
  #pragma unroll
        for (int kb = 0; kb < C::NB; ++kb)
  #pragma unroll
          for (int i = 0; i < 16; ++i) sacc[kb][i] *= c2;
      }
      float tmax = tile_max<C::NB>(sacc);
      if constexpr (POS) tmax *= c2;
      tmax = halves_max(tmax);
      const bool grow = tmax > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? tmax : m_run;
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
        m_run = m_new;
        l_run *= alpha;
  #pragma unroll
        for (int db = 0; db < C::DB; ++db)
  #pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
  #pragma unroll
      for (int kb = 0; kb < C::NB; ++kb)
  #pragma unroll
        for (int i = 0; i < 16; ++i) {
          if constexpr (POS) sacc[kb][i] = fast_exp2(fmaf(sacc[kb][i], c2, -m_use));
          else sacc[kb][i] = fast_exp2(sacc[kb][i] - m_use);
        }
      l_run += tile_sum<C::NB>(sacc);
  #pragma unroll
      for (int t = 0; t < BN / 16; ++t) {
        const f32x16& p = sacc[t >> 1];
        const int r0 = (t & 1) * 8;
        pk[t] = pack_bf16x8(p[r0 + 0], p[r0 + 1], p[r0 + 2], p[r0 + 3],
                            p[r0 + 4], p[r0 + 5], p[r0 + 6], p[r0 + 7]);
      }
    };

    // MFMA cluster of tile j: scores of tile j+1 from k_next (computed on the
    // wave's last tile too, from whatever the buffer holds, never used: one
    // code path) and O += V_j P_j; then the wait for this wave's copies of the
    // previous VALU cluster (only group 1 copies).
    auto mcluster = [&](int j, const uint8_t* k_next, const uint8_t* v_this) __attribute__((always_inline)) {
      if (j < ntw) {
        scores(k_next);
        pv(v_this);
        constexpr int kMfma = 0x008, kDsRead = 0x100;
        // Operand reads run a few MFMAs ahead: one K read per score MFMA,
        // then two transposing V reads per PV MFMA.
        __builtin_amdgcn_sched_group_barrier(kDsRead, 4, 0);
  #pragma unroll
        for (int i = 0; i < 2 * C::KS; ++i) {
          __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
        }
  #pragma unroll
        for (int i = 0; i < 4 * C::DB; ++i) {
          __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
        }
      }
      wait_dma();
    };

    wait_dma();
    __syncthreads();
    // Prologue: every wave forms P_0 from K_0.
    if (!SPLIT || ntw > 0) {
      scores(kl0);
      softmax(key_tile(0) * BN);
    }
    __syncthreads();
    // Group 1 starts one cluster later: its first slot copies K_2 into K_0's
    // buffer (free now) and waits for it; group 0 meanwhile runs M(0). With
    // SPLIT group 0 copies its own K_2 there too, waited for at the end of M(0).
    if (grp == 1) {
      copy_tile(KT{}, kl0, 2);
      wait_dma();
      __syncthreads();
    } else if (SPLIT) {
      copy_tile(KT{}, kl0, 2);
    }

    // Every wave runs the same clusters: M(j), barrier, V(j), barrier. With
    // group 1 one barrier behind, one wave of each SIMD is in an MFMA cluster
    // while the other is in a VALU cluster. V(j) is the softmax of tile j+1
    // and, for group 1, the copies of K_{j+3} (into K_{j+1}'s buffer) and
    // V_{j+2} (into V_j's), both last read by M(j) of the two groups.
    auto step = [&](auto ph, int j) __attribute__((always_inline)) {
      constexpr int P = decltype(ph)::value;   // j % 2
      const uint8_t* const k_next = P ? kl0 : kl1;   // K_{j+1}
      const uint8_t* const v_this = P ? vl1 : vl0;   // V_j
      uint8_t* const k_fill = P ? kl0 : kl1;         // K_{j+1}'s buffer, gets K_{j+3}
      uint8_t* const v_fill = P ? vl1 : vl0;         // V_j's buffer, gets V_{j+2}
      mcluster(j, k_next, v_this);
      __syncthreads();
      if (j + 1 < ntw) softmax(key_tile(j + 1) * BN);
      if (SPLIT || grp == 1) {
        copy_tile(KT{}, k_fill, j + 3);
        copy_tile(VT{}, v_fill, j + 2);
      }
      __syncthreads();
    };
    for (int j = 0; j < ns; j += 2) {
      step(std::integral_constant<int, 0>{}, j);
      if (j + 1 < ns) step(std::integral_constant<int, 1>{}, j + 1);
    }
    if (grp == 0) __syncthreads();
    wait_dma();
    // Every wave's copies have landed and every read is done: the four tile
    // buffers hold the 8 waves' O rows on their way out (8 KiB per wave).
    __syncthreads();

    if constexpr (SPLIT) {
      // Group 1 hands its reference max, its row-half sums and its O^T partials
      // to the group-0 wave with the same rows and lanes (through its own LDS
      // halves), which rescales both to the larger max and adds them.
      float* const xo = reinterpret_cast<float*>((w == 0 ? kl0 : w == 1 ? kl1 : w == 2 ? vl0 : vl1) + C::TILE);
      float* const xs = reinterpret_cast<float*>(vl1) + w * 128;
      if (grp == 1) {
  #pragma unroll
        for (int db = 0; db < C::DB; ++db)
  #pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4*>(xo + ((db * 4 + q4) * 64 + lane) * 4) =
                f32x4{oacc[db][4 * q4], oacc[db][4 * q4 + 1], oacc[db][4 * q4 + 2], oacc[db][4 * q4 + 3]};
        xs[lane] = m_run;
        xs[64 + lane] = l_run;
      }
      __syncthreads();
      if (grp == 1) return;
      const float m1 = xs[lane], l1 = xs[64 + lane];
      const float m = vmax(m_run, m1);
      const float mu = m == -INFINITY ? 0.f : m;
      const float a0 = fast_exp2(m_run - mu), a1 = fast_exp2(m1 - mu);
  #pragma unroll
      for (int db = 0; db < C::DB; ++db)
  #pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 p = *reinterpret_cast<const f32x4*>(xo + ((db * 4 + q4) * 64 + lane) * 4);
  #pragma unroll
          for (int e = 0; e < 4; ++e) oacc[db][4 * q4 + e] = fmaf(p[e], a1, oacc[db][4 * q4 + e] * a0);
        }
      l_run = fmaf(l1, a1, l_run * a0);
      m_run = m;
    }

    const float l_tot = halves_sum(l_run);
    {
      const float inv = 1.f / l_tot;
      u32x2 ov[C::DB][4];
  #pragma unroll
      for (int db = 0; db < C::DB; ++db)
  #pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          ov[db][g4] = u32x2{pack_bf16x2(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv),
                             pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
      uint8_t* const buf = blk < 2 ? kl0 : blk < 4 ? kl1 : blk < 6 ? vl0 : vl1;
      store_rows_staged<D>(O + off + (size_t)qw * D, N - qw, buf + (blk & 1) * 32 * RB, ov, lane);
    }
    if (qrow < N && hi == 0) LSE[(size_t)head * N + qrow] = (m_run + fast_log2(l_tot)) * kLn2;
  };
  if constexpr (PAIR) {
    // Two causal query tiles, the heavy ntq-1-u and then the light u: every
    // pair has the same number of key tiles (the middle tile of an odd count
    // is alone).
    const int qa = ntq - 1 - rank, qb = rank;
    item(qa);
    if (qb != qa) {
      __syncthreads();
      item(qb);
    }
  } else {
    item(CAUSAL ? (ntq - 1 - rank) : rank);
  }
}

template <bool CAUSAL, bool POS, bool SPLIT = false, bool PAIR = false>
static hipError_t launch_fwd_pp(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                uint16_t* o, float* lse, int BH, int N, float scale,
                                hipStream_t stream) {
  const int bmq = SPLIT ? 128 : PingPongCfg::BM;
  const int ntq = (N + bmq - 1) / bmq;
  const int xcd_group = (BH % 8 == 0) ? BH / 8 : 0;
  const float c2 = scale * kLog2e;
  const int units = PAIR ? (ntq + 1) / 2 : ntq;   // workgroups per head
  dim3 grid((unsigned)(units * BH)), block(PingPongCfg::THREADS);
  hipLaunchKernelGGL((fa_fwd_pp_kernel<CAUSAL, POS, SPLIT, PAIR>), grid, block, 0, stream,
                     q, k, v, o, lse, BH, N, ntq, c2, xcd_group);
  return hipGetLastError();
}

// Long d = 128 sequences (on average at least ~64 key tiles per query tile)
// with at least one 256-row workgroup per CU take the two-group kernel:
// measured 3-5 % faster there (B=1, H=16, N=16384 causal; N=8192 causal and
// not; B=2, H=32, N=4096 non-causal), but 5-14 % slower on shorter causal
// sequences (N = 4096, 2048), where its 256-row workgroups leave SIMDs idle
// across a 4-tile diagonal that a second, independent workgroup would fill.
// d = 128 grids of at most 256 128-row query tiles (one per CU) with at least
// 1024 keys take the two-group kernel with the keys split between the groups:
// measured 11-15 % faster causal (B=1 with H=8, N=4096; H=4, N=8192; H=2,
// N=16384) and 2-5 % non-causal (H=8, N=4096; H=2, N=16384). With 512 tiles
// (B=2, H=16, N=2048) the split kernel needs two rounds and is 11 % slower.
bool fwd_uses_split_kernel(int BH, int N, int d) {
  return d == 128 && N >= 1024 && (long)((N + 127) / 128) * BH <= 256;
}

bool fwd_uses_two_group_kernel(int BH, int N, int d, bool causal) {
  return d == 128 && (long)((N + PingPongCfg::BM - 1) / PingPongCfg::BM) * BH >= 256 &&
         N >= (causal ? 8192 : 4096);
}

// Causal d = 128 grids of 257-512 128-row query tiles with at least 4096
// keys take the split-key two-group kernel with two query tiles per
// workgroup (heavy, then light): one round of at most 256 workgroups, each
// with the same number of key tiles. Measured against the kernel they took
// before (fa_fwd_kernel below N = 8192, fa_fwd_pp_kernel from it): -5 to
// -8 % at N = 4096 (B*H = 12, 16), -18 to -26 % at N = 8192 (B*H = 6, 8),
// -20 to -30 % at N = 16384 (B*H = 3, 4); but +5 % at N = 2048 (B*H = 32,
// the fwd+bwd workload's shape) and +24 % at N = 1024, where each tile's
// start-up and merge weigh more, and +7 to +24 % on grids of more than 512
// tiles (two rounds).
bool fwd_uses_paired_split(int BH, int N, int d, bool causal) {
  const long tiles = (long)((N + 127) / 128) * BH;
  return d == 128 && causal && N >= 4096 && tiles > 256 && tiles <= 512;
}

hipError_t fwd_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        uint16_t* o, float* lse, int BH, int N, int d, float scale,
                        bool causal, hipStream_t stream) {
  const bool pos = scale > 0.f;
  if (fwd_uses_paired_split(BH, N, d, causal)) {
    if (pos) return launch_fwd_pp<true, true, true, true>(q, k, v, o, lse, BH, N, scale, stream);
    return launch_fwd_pp<true, false, true, true>(q, k, v, o, lse, BH, N, scale, stream);
  }
  if (fwd_uses_split_kernel(BH, N, d)) {
    if (causal && pos) return launch_fwd_pp<true, true, true>(q, k, v, o, lse, BH, N, scale, stream);
    if (!causal && pos) return launch_fwd_pp<false, true, true>(q, k, v, o, lse, BH, N, scale, stream);
    if (causal && !pos) return launch_fwd_pp<true, false, true>(q, k, v, o, lse, BH, N, scale, stream);
    return launch_fwd_pp<false, false, true>(q, k, v, o, lse, BH, N, scale, stream);
  }
  if (fwd_uses_two_group_kernel(BH, N, d, causal)) {
    if (causal && pos) return launch_fwd_pp<true, true>(q, k, v, o, lse, BH, N, scale, stream);
    if (!causal && pos) return launch_fwd_pp<false, true>(q, k, v, o, lse, BH, N, scale, stream);
    if (causal && !pos) return launch_fwd_pp<true, false>(q, k, v, o, lse, BH, N, scale, stream);
    return launch_fwd_pp<false, false>(q, k, v, o, lse, BH, N, scale, stream);
  }
#define FA_FWD_CASE(DD, CC, PP) \
  if (d == DD && causal == CC && pos == PP) \
    return launch_fwd<DD, CC, PP>(q, k, v, o, lse, BH, N, scale, stream);
  FA_FWD_CASE(128, true, true)
  FA_FWD_CASE(128, false, true)
  FA_FWD_CASE(64, true, true)
  FA_FWD_CASE(64, false, true)
  FA_FWD_CASE(128, true, false)
  FA_FWD_CASE(128, false, false)
  FA_FWD_CASE(64, true, false)
  FA_FWD_CASE(64, false, false)
#undef FA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
