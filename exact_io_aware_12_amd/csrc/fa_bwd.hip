// Backward pass of fused exact attention for gfx950.
//
// Method: "FlashAttention core principles" (lesson 1), section 5: only one
// statistic per row is kept from the forward pass; S and P are recomputed tile
// by tile, and per tile pair dV += P^T dO, dP = dO V^T,
// dS = P o (dP - D) (times the scale), dQ += dS K, dK += dS^T Q. The row
// statistic D_i = sum_j P_ij dP_ij is a sum over the WHOLE row (it equals
// dO_i . O_i); taken per tile it would not be the gradient, so it is computed
// once per row before the tile loops.
//
// Two kernels on the caller's stream:
//   1. fa_bwd_dq:    D_i = dO_i . O_i (written out) and dQ. One workgroup per
//      128-query tile (4 wave64s x 32 queries, two workgroups per CU); the
//      loop runs over 64-key tiles and recomputes S and dP (inner loop over
//      K/V, so dQ stays in registers). When the causal grid fits in one
//      round, each workgroup instead holds two such groups of 4 waves that
//      take alternate key tiles of the same query tile, and their partial
//      dQ are summed in LDS: the round is bound by the longest tile's chain
//      of key tiles, which this halves.
//   2. fa_bwd_dkdv:  dK and dV. One workgroup per key tile pair (8 wave64s,
//      two per SIMD: 4 key blocks of 32 x 2 query halves); the loop runs over
//      64-query tiles (outer loop over K/V, inner over Q, so dK and dV stay
//      in registers). The two query halves are two groups of 4 waves that
//      take turns, one barrier apart: while one wave of a SIMD runs its MFMA
//      cluster (dV, dK of the previous query tile, then S, dP of this one),
//      the other runs its VALU cluster (P and dS of its current tile).
// Splitting dQ from dK/dV costs two extra matmuls per tile pair (S and dP are
// computed in both kernels: 7 instead of 5), and buys the removal of every
// cross-workgroup accumulation: on this multi-XCD device, device-scope fp32
// atomics into a dQ accumulator are performed past the L2 and cost more than
// the recomputation.
//
// gfx950 mapping (32x32x16 bf16 MFMAs, fp32 accumulate):
//   * dK/dV kernel: S = Q K^T and dP = dO V^T are computed with one key per
//     lane (the B operands are this wave's 32 rows of the key tile's K and V,
//     staged in LDS once per key tile), so P and dS sit in registers in
//     exactly the layout the B operand of dV^T += dO^T P and
//     dK^T += Q^T dS needs (k-slots are queries). Q and dO tiles go from
//     HBM/L2 straight into LDS (global_load_lds_dwordx4, a ring of three) in
//     one XOR swizzle that serves both the row-major operand reads of S and
//     dP (ds_read_b128) and the transposing reads that give Q^T and dO^T
//     (ds_read_b64_tr_b16) without bank conflicts. Each lane loads one
//     row's LSE and D; DPP row broadcasts hand every accumulator element its
//     row's values.
//   * dQ kernel: the transposed form of the forward pass, one query per lane:
//     S^T = K Q^T and dP^T = V dO^T (Q and dO rows in registers as B
//     operands, K and V rows from LDS), P^T and dS^T element-wise with the
//     lane's own LSE and D, and dQ^T += K^T dS^T with dS^T fed from the
//     accumulator registers as the B operand and K^T from transposing reads
//     of the same swizzled K tile.
//   * dQ kernel: scheduling-group barriers interleave the MFMAs with the VALU
//     work and the LDS operand reads of each phase. dK/dV kernel: its MFMA
//     cluster is an explicit software pipeline (operands read a fixed number
//     of MFMAs ahead, the order pinned by scheduling barriers).
#include <mutex>
#include <type_traits>
#include <utility>

#include "fa_common.h"

namespace fa {

// ----------------------------------------------------------------- dK, dV
#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct BwdCfg {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BNK = 128;          // keys per workgroup: 4 key blocks of 32
  static constexpr int BMQ = 64;           // queries per step: 2 halves of 32
  static constexpr int RB = D * 2;         // bytes per Q / dO / V row in LDS
  static constexpr int QTILE = BMQ * RB;   // 16 KiB (d=128)
  static constexpr int VTILE = BNK * RB;   // 32 KiB (d=128): one K or V key tile
  static constexpr int QLOADS = QTILE / 1024 / WAVES;   // 1 KiB copies per wave
  static constexpr int VLOADS = VTILE / 1024 / WAVES;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int PREFETCH = 4;       // MFMAs whose LDS operands are in flight
  // A ring of three Q and three dO tiles plus one K and one V key tile: the
  // whole 160 KiB of a CU's LDS at d = 128.
  static_assert(6 * QTILE + 2 * VTILE <= 160 * 1024, "LDS");
  // The partial dK (then dV) sums of group 1 go through the Q / dO buffers.
  static_assert(4 * 16 * DB * 64 * 4 <= 6 * QTILE, "partial sums fit the Q/dO buffers");
  // The bf16 gradients are staged row-major in the K and V tiles.
  static_assert(BNK * RB <= VTILE && (BNK * RB / 16) % THREADS == 0, "staging");
};

// Swizzled byte offset of 2-byte element (row, col) in a tile with R-byte
// rows. Chunks of 16 bytes are XORed with a function of the row that is a
// bijection over 16 consecutive rows (so a row-major operand read of 16 rows
// hits 16 distinct bank groups) and whose top bits follow row%4 (so the 4
// rows of a transposing read fall in 4 distinct 64-byte bank quarters).
template <int R>
__device__ __forceinline__ int sw_xor(int row) {
  if constexpr (R == 256) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}
template <int R>
__device__ __forceinline__ int sw_off(int row, int col) {
  const int byte = col * 2;
  return row * R + ((((byte >> 4) ^ sw_xor<R>(row))) << 4) + (byte & 15);
}

// Global -> LDS copies (global_load_lds: lane i writes LDS bytes
// [M0 + size*i, +size)). They are issued from an asm statement so that the
// compiler does not treat them as LDS stores that may alias the reads of the
// other buffer (it would then wait for every copy before the next LDS read);
// completion is awaited explicitly with wait_vmem() before the barrier that
// publishes a buffer. The s_nop covers the M0-write -> LDS-DMA hazard.
// The statements below write M0, which the compiler reserves; declaring the
// clobber is what tells it so (it warns that a reserved register is listed,
// hence the local pragma). Nothing else in this file uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds_addr) : "memory", "m0");
  strict_copy_wait();
}
// Scalar-base form: the tile's base address is one SGPR pair and each lane
// adds a 32-bit byte offset (no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void lds_copy16s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
  strict_copy_wait();
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS void*)p;
}

// This wave's share of the copy of LOADS*WAVES KiB of rows x D bf16 (rows past
// N read row N-1) from global memory into a swizzled LDS tile: lane i of each
// 1 KiB copy writes LDS bytes [16i, 16i+16), so it fetches the chunk the
// swizzle puts there.
template <int D, int LOADS>
__device__ __forceinline__ void dma_rows(const uint16_t* __restrict__ src, const uint8_t* lds,
                                         int row0, int N, int w, int lane) {
  constexpr int R = D * 2, RPL = 1024 / R, CPR = R / 16;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int lrow = (w * LOADS + i) * RPL;
    const int row = lrow + lane / CPR;
    const int c = (lane % CPR) ^ sw_xor<R>(row);
    const uint16_t* g = src + (size_t)min(row0 + row, N - 1) * D + c * 8;
    lds_copy16(g, lds_addr(lds + lrow * R));
  }
}

__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // s_waitcnt vmcnt(0)
}

// Two transposing reads -> one bf16x8 MFMA operand: k-slot s of half h is
// row 8*(s/4) + 4h + s%4 of the 16 rows read. o0 / o1 are the byte offsets
// of the two halves (the swizzle depends on bits 2-3 of the row, so the half
// 8 rows further has its own offset); base adds multiples of 16 rows.
__device__ __forceinline__ bf16x8 tr_operand(const uint8_t* base, int o0, int o1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(base + o0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(base + o1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// DPP row broadcast: every lane receives the value of lane I of its 16-lane
// row (row_newbcast).
template <int I>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + I, 0xF, 0xF, true));
}
// f(integral_constant<int, I>) for each I of the sequence, in order.
template <typename F, int... I>
__device__ __forceinline__ void static_for(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

// dK, dV for one key tile (or a causal pair of them) per workgroup. The two
// query halves of each 64-query tile are two groups of 4 waves (group g =
// waves 4g .. 4g+3; waves w and w+4 share a SIMD) that alternate two
// clusters per query tile s:
//   M(s): dV^T += dO_{s-1}^T P_{s-1} and dK^T += Q_{s-1}^T dS_{s-1} (4*DB
//         MFMAs, from the packed P / dS of the previous tile), then S and dP
//         of tile s (2*KS MFMAs): MFMAs and LDS operand reads only;
//   V(s): P = exp2(S*scale*log2e - LSE*log2e) and dS = P o (dP - D) of tile s,
//         packed to bf16: VALU work only.
// Group 1 runs one workgroup barrier behind group 0, so while one wave of a
// SIMD issues MFMAs the other issues VALU work. Q / dO tiles live in a ring
// of three LDS buffers: in V(s), after both groups' M(s) have read tile s-1,
// group 1 copies tile s+2 into its buffers, and it waits for the copies at
// the end of its M(s+1), before the barrier that lets group 0 read them.
// The two groups' partial dK / dV are summed in LDS at the end of a key tile.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dvec,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    int BH, int N, int nunits, float c2, float scale, int xcd_group) {
  using C = BwdCfg<D>;
  constexpr int KS = C::KS, DB = C::DB, RB = C::RB;
  constexpr int GLOADS = C::QTILE / 1024 / 4;   // 1 KiB copies per wave of group 1, per tile
  // Q tiles in buffers 0-2, dO tiles in 3-5 (a ring of three query tiles),
  // this key tile's K and V; at the end of a key tile the first bytes of the
  // ring carry the partial dK / dV sums.
  __shared__ __attribute__((aligned(1024))) uint8_t qo_lds[6 * C::QTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[C::VTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[C::VTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  // Wave w: keys 32*kb .. +31 of the key tile, queries 32*qh .. +31 of each
  // query tile; qh is the wave's group. Waves w and w+4 share a SIMD.
  const int kb = w & 3, qh = w >> 2;

  // Workgroup -> (head, work unit). Causal: unit u covers the key tiles u and
  // nkt-1-u: first key tile u with the query tiles in descending order, then
  // key tile nkt-1-u with them in ascending order. Every unit then costs the
  // same number of query-tile steps, and since the units of a head start
  // together, they all work on the same query tile (or two) at any time, so
  // the Q / dO tiles being read stay in the XCD's L2. Non-causal: one key
  // tile per unit, ascending.
  int head, unit;
  {
    const int b = blockIdx.x;
    if (xcd_group > 0) {
      // Workgroups are dispatched round-robin over the 8 XCDs; XCD x gets the
      // heads [x*G, (x+1)*G), head-major.
      const int x = b & 7, s = b >> 3;
      head = x * xcd_group + s / nunits;
      unit = s % nunits;
    } else {
      head = b / nunits;
      unit = b % nunits;
    }
  }
  const size_t off = (size_t)head * N * D;
  const uint16_t* Qh = Q + off;
  const uint16_t* dOh = dO + off;
  const float* LSEh = LSE + (size_t)head * N;
  const float* Dh = Dvec + (size_t)head * N;
  const int nqt = (N + C::BMQ - 1) / C::BMQ;

  // Per-lane LDS byte offsets, k-step / block 0. The swizzle only moves
  // 16-byte chunks within a row, so the other k-steps and 32-column blocks
  // are XORs of these (k-step ks: ^ ks << 5 for row-major reads; block db:
  // ^ db << 6 for transposing reads, and the half 8 rows on: ^ 32, + 8 rows),
  // one register each instead of one per (k-step, block, half).
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int rq0 = sw_off<RB>(l32, 8 * hi);
  const int tq0 = sw_off<RB>(tr_row, tr_col);

  f32x16 dkacc[DB], dvacc[DB];
  f32x16 sacc, pacc;        // S and dP of the current query tile (this wave's 32 x 32)
  bf16x8 pbv[2], sbv[2];    // packed P and dS of the previous query tile

  const int nkt_ = (N + C::BNK - 1) / C::BNK;
  const int nparts = (CAUSAL && 2 * unit + 1 != nkt_) ? 2 : 1;
  for (int part = 0; part < nparts; ++part) {
    const int kt = part == 0 ? unit : nkt_ - 1 - unit;
    const int k0 = kt * C::BNK;
    const int kk = k0 + 32 * kb + l32;
    const bool rev = CAUSAL && part == 0;
    const int it_lo = CAUSAL ? (k0 / C::BMQ) : 0;
    const int nsteps = nqt - it_lo;
    auto tile_at = [&](int step) __attribute__((always_inline)) {
      return rev ? nqt - 1 - step : it_lo + step;
    };
    auto qbuf = [&](int b) __attribute__((always_inline)) { return qo_lds + b * C::QTILE; };
    auto obuf = [&](int b) __attribute__((always_inline)) { return qo_lds + (3 + b) * C::QTILE; };
    // Group 1's copy of query tile `step` (Q and dO) into buffer b: wave kb
    // copies rows 16kb .. 16kb+15 (GLOADS KiB); tiles past the last repeat
    // it (in bounds, unused), rows past N read row N-1.
    auto copy_tile = [&](int step, int b) __attribute__((always_inline)) {
      const int row0 = tile_at(min(step, nsteps - 1)) * C::BMQ;
      constexpr int RPL = 1024 / RB, CPR = RB / 16;
      const bool full = row0 + C::BMQ <= N;
#pragma unroll
      for (int i = 0; i < GLOADS; ++i) {
        const int lrow = (kb * GLOADS + i) * RPL;
        const int row = lrow + lane / CPR;
        const int c = (lane % CPR) ^ sw_xor<RB>(row);
        const int src_row = full ? row0 + row : min(row0 + row, N - 1);
        // Unsigned: src_row * RB reaches 2^32 - RB when N * d approaches the
        // entry points' 2^31 - 1 limit (B = H = 1), past the int range.
        const uint32_t voff = (uint32_t)src_row * (uint32_t)RB + (uint32_t)(c * 16);
        lds_copy16s(Qh, voff, lds_addr(qbuf(b) + lrow * RB));
        lds_copy16s(dOh, voff, lds_addr(obuf(b) + lrow * RB));
      }
    };

    // -LSE*log2(e) and D of this wave's rows of tile `step`, one row per
    // lane: lane l holds row 8*((l%16)/4) + 4*(l/32) + l%4, which is the row
    // of accumulator element l%16 in lane l's half of the wave, so element i
    // takes its value from lane i of its 16-lane row (a DPP broadcast). Rows
    // past N read row N-1 (their P is zero). Issued at the start of the MFMA
    // cluster, used in the VALU cluster (tile 0's: with the prologue copies).
    float nlse_l, d_l;
    const int srow = 8 * ((lane & 15) >> 2) + 4 * hi + (lane & 3);
    auto load_stats = [&](int step) __attribute__((always_inline)) {
      const int r = min(tile_at(step) * C::BMQ + 32 * qh + srow, N - 1);
      nlse_l = LSEh[r];
      d_l = Dh[r];
    };
    // Prologue: this key tile's K and V, query tiles 0 and 1 (all waves).
    dma_rows<D, C::VLOADS>(K + off, k_lds, k0, N, w, lane);
    dma_rows<D, C::VLOADS>(V + off, v_lds, k0, N, w, lane);
    dma_rows<D, C::QLOADS>(Qh, qbuf(0), tile_at(0) * C::BMQ, N, w, lane);
    dma_rows<D, C::QLOADS>(dOh, obuf(0), tile_at(0) * C::BMQ, N, w, lane);
    if (nsteps > 1) {
      dma_rows<D, C::QLOADS>(Qh, qbuf(1), tile_at(1) * C::BMQ, N, w, lane);
      dma_rows<D, C::QLOADS>(dOh, obuf(1), tile_at(1) * C::BMQ, N, w, lane);
    }
    load_stats(0);
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      dkacc[i] = zero16();
      dvacc[i] = zero16();
    }
    wait_vmem();
    __syncthreads();

    // P and dS of tile `step` from sacc / pacc, packed (registers 8t .. 8t+7:
    // the k-slot order of the dV / dK B operands).
    auto valu = [&](int step) __attribute__((always_inline)) {
      const int qw = tile_at(step) * C::BMQ + 32 * qh;
      const float nl = nlse_l * -kLog2e;
      static_for([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        sacc[i] = fmaf(sacc[i], c2, row_bcast<i>(nl));
        pacc[i] = pacc[i] - row_bcast<i>(d_l);
      }, std::make_integer_sequence<int, 16>{});
      const bool masked = (CAUSAL && qw < kk - l32 + 31) || qw + 32 > N || k0 + C::BNK > N;
      if (masked) {
        // Element i holds query qw + 4hi + c_i (c_i = 8(i/4) + i%4): masked
        // when the key is above it (causal), or it or the key is past N.
        const int qd = kk - qw - 4 * hi, qr = N - qw - 4 * hi;
        const bool kout = kk >= N;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ci = 8 * (i >> 2) + (i & 3);
          sacc[i] = ((CAUSAL && qd > ci) || kout || ci >= qr) ? -INFINITY : sacc[i];
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float pv[8], dv8[8];
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int g4 = 2 * t + g2;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = fast_exp2(sacc[4 * g4 + e]);
            pv[4 * g2 + e] = p;
            dv8[4 * g2 + e] = p * pacc[4 * g4 + e];
          }
        }
        pbv[t] = pack_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
        sbv[t] = pack_bf16x8(dv8[0], dv8[1], dv8[2], dv8[3], dv8[4], dv8[5], dv8[6], dv8[7]);
      }
    };

    // The MFMA cluster as an explicit software pipeline: MFMAs 0 .. NDV-1
    // are dV^T / dK^T of the previous tile (A: transposing reads of dO / Q at
    // atb, B: the packed P / dS), then 2*KS MFMAs are S and dP of the current
    // tile in k-step pairs (A: Q / dO rows at aqb, B: K / V rows at ak). The
    // operands of MFMA i + PREFETCH are read before MFMA i is issued, and
    // scheduling barriers keep that order (left to itself, the scheduler may
    // spend the look-ahead on reads needed much later).
    auto mcluster = [&](auto with_dvdk, auto with_sdp, int atb, int aqb, int ak) __attribute__((always_inline)) {
      constexpr int NDV = decltype(with_dvdk)::value ? 4 * DB : 0;
      constexpr int NM = NDV + (decltype(with_sdp)::value ? 2 * KS : 0);
      constexpr int PF = C::PREFETCH;
      bf16x8 opa[PF + 1], opb[PF + 1];
      auto fetch = [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        constexpr int r = i % (PF + 1);
        if constexpr (i < NDV) {
          constexpr int t = i / (2 * DB), db = (i / 2) % DB, isk = i % 2;
          const int o0 = atb ^ (db << 6), o1 = (o0 ^ 32) + 8 * RB;
          opa[r] = tr_operand((isk ? qbuf(0) : obuf(0)) + 16 * t * RB, o0, o1);
        } else {
          constexpr int j = i - NDV, ks = j / 2, isp = j % 2;
          const int oq = aqb ^ (ks << 5), ok = ak ^ (ks << 5);
          opa[r] = *reinterpret_cast<const bf16x8*>((isp ? obuf(0) : qbuf(0)) + oq);
          opb[r] = *reinterpret_cast<const bf16x8*>((isp ? v_lds : k_lds) + ok);
        }
      };
      auto mfma_i = [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        constexpr int r = i % (PF + 1);
        if constexpr (i < NDV) {
          constexpr int t = i / (2 * DB), db = (i / 2) % DB, isk = i % 2;
          if constexpr (isk) dkacc[db] = mfma_32x32x16(opa[r], sbv[t], dkacc[db]);
          else dvacc[db] = mfma_32x32x16(opa[r], pbv[t], dvacc[db]);
        } else {
          constexpr int j = i - NDV, isp = j % 2;
          if constexpr (j < 2) {
            if constexpr (isp) pacc = mfma_32x32x16(opa[r], opb[r], zero16());
            else sacc = mfma_32x32x16(opa[r], opb[r], zero16());
          } else {
            if constexpr (isp) pacc = mfma_32x32x16(opa[r], opb[r], pacc);
            else sacc = mfma_32x32x16(opa[r], opb[r], sacc);
          }
        }
      };
      static_for([&](auto ic) __attribute__((always_inline)) {
        if constexpr (decltype(ic)::value < NM) fetch(ic);
      }, std::make_integer_sequence<int, PF>{});
      __builtin_amdgcn_sched_barrier(0);
      static_for([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + PF < NM) fetch(std::integral_constant<int, i + PF>{});
        mfma_i(ic);
        __builtin_amdgcn_sched_barrier(0);
      }, std::make_integer_sequence<int, NM>{});
    };

    // Prologue: every wave forms S, dP and then P, dS of tile 0.
    mcluster(std::false_type{}, std::true_type{}, 0, rq0 + 32 * qh * RB, rq0 + 32 * kb * RB);
    valu(0);
    __syncthreads();
    // Group 1 starts one barrier later: its first slot copies tile 2.
    if (qh == 1) {
      if (nsteps > 2) copy_tile(2, 2);
      wait_vmem();
      __syncthreads();
    }

    // Step s (1 .. nsteps): M(s), barrier, V(s), barrier. Tile s sits in
    // buffer s % 3, tile s-1 in (s-1) % 3, which then receives tile s+2. The
    // last step (no tile s) only finishes dV, dK of tile s-1.
    auto step = [&](auto last, int s, int p, int prev) __attribute__((always_inline)) {
      constexpr bool LAST = decltype(last)::value;
      // Buffer b's bytes start b * QTILE after buffer 0's (a multiple of 16
      // KiB, above the bits the XORs touch). The offsets are re-derived in
      // every step (an empty asm hides that they do not change), so that
      // three registers stay live across the loop rather than one per
      // (k-step, operand).
      int aq = rq0 + 32 * qh * RB, ak = rq0 + 32 * kb * RB, at = tq0 + 32 * qh * RB;
      asm volatile("" : "+v"(aq), "+v"(ak), "+v"(at));
      if constexpr (!LAST) load_stats(s);
      mcluster(std::true_type{}, std::integral_constant<bool, !LAST>{}, at + prev * C::QTILE,
               aq + p * C::QTILE, ak);
      // No instruction crosses the cluster boundaries (the scheduler would
      // otherwise hoist the start of the VALU cluster above the barrier, into
      // the MFMA cluster, where it waits on the statistics loads).
      wait_vmem();
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!LAST) valu(s);
      if (qh == 1 && s + 2 < nsteps) copy_tile(s + 2, prev);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    int p = 1, prev = 0;
    for (int s = 1; s < nsteps; ++s) {
      step(std::false_type{}, s, p, prev);
      prev = p;
      p = p == 2 ? 0 : p + 1;
    }
    step(std::true_type{}, nsteps, p, prev);
    if (qh == 0) __syncthreads();

    // ---- Sum the two groups' partial dK^T, dV^T and store them. For each
    // gradient: group 1 writes its partial into the Q / dO ring (fp32,
    // lane-contiguous 16-byte chunks: conflict-free); group 0 adds it to its
    // own, scales (dK = scale * dK^T), rounds to bf16 and writes the rows
    // row-major into the K (dK) or V (dV) tile, 16-byte chunks XOR-swizzled
    // by the row so that a wave's 32 rows spread over the banks; then all 8
    // waves store whole rows, 16 bytes per lane (coalesced). Group 1 writes
    // the dV partial while dK is being stored. Every LDS read of this key
    // tile finished before the last barrier, and no copy is in flight.
    {
      constexpr int CPR = RB / 16;                 // 16-byte chunks per row
      // The lane indices are re-derived here (an empty asm hides that they
      // are the kernel's), so that no address of this phase is computed
      // early and held across the query-tile loop.
      int t_id = tid;
      asm volatile("" : "+v"(t_id));
      const int ln = t_id & 63;
      f32x4* part_w = reinterpret_cast<f32x4*>(qo_lds) + kb * (DB * 4 * 64) + ln;
      const int row = 32 * kb + (ln & 31);         // this lane's row of the key tile
      const int hh = ln >> 5;
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        f32x16 (&acc)[DB] = which == 0 ? dkacc : dvacc;
        uint8_t* stage = which == 0 ? k_lds : v_lds;
        if (qh == 1) {
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
              part_w[(db * 4 + g4) * 64] = f32x4{acc[db][4 * g4], acc[db][4 * g4 + 1],
                                                 acc[db][4 * g4 + 2], acc[db][4 * g4 + 3]};
        }
        __syncthreads();
        if (qh == 0) {
          const float sc = which == 0 ? scale : 1.f;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const f32x4 o = part_w[(db * 4 + g4) * 64];
              const int c = (4 * db + g4) ^ (row & (CPR - 1));
              *reinterpret_cast<u32x2*>(stage + row * RB + c * 16 + 8 * hh) =
                  u32x2{pack_bf16x2((acc[db][4 * g4] + o[0]) * sc, (acc[db][4 * g4 + 1] + o[1]) * sc),
                        pack_bf16x2((acc[db][4 * g4 + 2] + o[2]) * sc, (acc[db][4 * g4 + 3] + o[3]) * sc)};
            }
        }
        __syncthreads();
        uint16_t* dst = (which == 0 ? dK : dV) + off;
#pragma unroll
        for (int j = 0; j < C::BNK * CPR / C::THREADS; ++j) {
          const int idx = t_id + j * C::THREADS;
          const int r = idx / CPR, c = idx % CPR;
          const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * RB + ((c ^ (r & (CPR - 1))) * 16));
          if (k0 + r < N) *reinterpret_cast<u32x4*>(dst + (size_t)(k0 + r) * D + c * 8) = v;
        }
      }
      __syncthreads();
    }
  }
}

// ----------------------------------------------------------------- dQ (and D)
template <int D>
struct DqCfg {
  static constexpr int BM = 128;              // queries per workgroup (32 per wave)
  static constexpr int THREADS = 256;         // 4 waves per key-tile group
  static constexpr int BN = 64;               // keys per tile
  static constexpr int RB = D * 2;            // bytes per K / V row in LDS
  static constexpr int TILE = BN * RB;        // 16 KiB (d=128)
  static constexpr int LOADS = TILE / 1024 / 4;   // 1 KiB copies per wave
  static constexpr int NB = BN / 32;          // 32-key blocks per tile
  static constexpr int DB = D / 32;           // 32-wide head-dim blocks
  static constexpr int KS = D / 16;           // k-steps of S^T and dP^T
  static_assert(KS == 2 * LOADS, "one K or V copy per k-step of the first block");
};

// dQ_i = scale * sum_j dS_ij K_j for one 128-query tile per workgroup.
template <int D, bool CAUSAL, int G>
__global__ __launch_bounds__(256 * G) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ O, const float* __restrict__ LSE, float* __restrict__ Dvec,
    uint16_t* __restrict__ dQ, int BH, int N, int ntq, float c2, float scale, int xcd_group) {
  using C = DqCfg<D>;
  constexpr int KS = C::KS, DB = C::DB, NB = C::NB, RB = C::RB;
  // G groups of 4 waves share the query tile and split its key tiles (group
  // g takes tiles g, g+G, ...), each with its own double buffer.
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[G][2][C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[G][2][C::TILE];
  // With two groups (one workgroup per CU) the tile's O rows, for D, are
  // staged in the LDS that the K / V buffers leave free.
  __shared__ __attribute__((aligned(1024))) uint8_t o_lds[G == 2 ? 2 * C::TILE : 16];
  static_assert(G == 1 || (2 * G * 2 + 2) * C::TILE <= 160 * 1024, "LDS");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wall = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = G == 1 ? 0 : wall >> 2;   // key-tile group
  const int w = wall & 3;              // wave within the group (its 32 query rows)
  const int l32 = lane & 31, hi = lane >> 5;

  // Workgroup -> (head, query tile): heaviest causal tiles first, the
  // workgroups of a head on one XCD (as in the forward pass).
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
  const int qt = CAUSAL ? (ntq - 1 - rank) : rank;
  const int q0 = qt * C::BM;
  const int qw = q0 + 32 * w;          // first query row of this wave
  const int qrow = qw + l32;           // this lane's query row
  const int qc = min(qrow, N - 1);     // rows past N compute with row N-1 (never stored)
  const size_t off = (size_t)head * N * D;
  const int kend = CAUSAL ? min(N, q0 + C::BM) : N;
  const int nt = (kend + C::BN - 1) / C::BN;
  // Key tiles this wave computes: 0 .. ntw-1 (causal waves stop at the diagonal).
  const int ntw = CAUSAL ? min(nt, (min(N, qw + 32) + C::BN - 1) / C::BN) : nt;

  dma_rows<D, C::LOADS>(K + off, k_lds[grp][0], min(grp, nt - 1) * C::BN, N, w, lane);
  dma_rows<D, C::LOADS>(V + off, v_lds[grp][0], min(grp, nt - 1) * C::BN, N, w, lane);
  // The tile's Q rows (and, with two groups, its dO and O rows) go to LDS by
  // coalesced copies, 64 rows per buffer, Q and dO into the second buffers
  // (free until the first step's copies): loaded one row per lane, every
  // 16-byte load would be spread over 32 rows. Rows past N read row N-1.
  if constexpr (G == 2) {
    dma_rows<D, C::LOADS>(Q + off, k_lds[grp][1], q0 + 64 * grp, N, w, lane);
    dma_rows<D, C::LOADS>(dO + off, v_lds[grp][1], q0 + 64 * grp, N, w, lane);
    dma_rows<D, C::LOADS>(O + off, o_lds + grp * C::TILE, q0 + 64 * grp, N, w, lane);
  } else {
    dma_rows<D, C::LOADS>(Q + off, k_lds[0][1], q0, N, w, lane);
    dma_rows<D, C::LOADS>(Q + off, v_lds[0][1], q0 + 64, N, w, lane);
  }

  // This lane's Q and dO rows as B operands (k-slots = head dim), read from
  // the staged tiles after the first barrier (with one group, dO straight
  // from memory), and its row statistics: LSE in log2 units and D = dO . O
  // (B1), summed over the lane's half of the row and exchanged with the
  // other half. D is also written out for the dK / dV kernel, which runs
  // after this one. With one group the O row chunks load meanwhile.
  bf16x8 qreg[KS], doreg[KS];
  u32x4 oreg[KS];
  if constexpr (G == 1) {
    const size_t o = off + (size_t)qc * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      oreg[ks] = ld_global_16B(O + o + ks * 16);
      doreg[ks] = __builtin_bit_cast(bf16x8, ld_global_16B(dO + o + ks * 16));
    }
  }
  const float nlse2 = -LSE[(size_t)head * N + qc] * kLog2e;
  float drow = 0.f;

  // Per-lane LDS offsets (the swizzle only looks at bits 0-3 of the row, so
  // 16- and 32-row steps are immediates): row-major reads of row l32 (K and
  // V operands of S^T and dP^T), transposing reads (K^T operand of dQ^T).
  int rk_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) rk_off[ks] = sw_off<RB>(l32, 16 * ks + 8 * hi);
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int tk_off[2][DB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < DB; ++db) tk_off[h][db] = sw_off<RB>(tr_row + 8 * h, 32 * db + tr_col);

  f32x16 dqacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dqacc[i] = zero16();

  // Per-lane byte offsets of this wave's K / V tile copies (lane i of copy c
  // writes LDS bytes [16i, 16i+16) of 1 KiB block w*LOADS+c, so it fetches
  // the chunk the swizzle puts there), for a full tile and for the ragged
  // last tile (rows past N read row N-1).
  uint32_t offd[C::LOADS], offr[C::LOADS];
  {
    constexpr int RPL = 1024 / RB, CPR = RB / 16;
    const int kl = (N - 1) / C::BN * C::BN;
#pragma unroll
    for (int c = 0; c < C::LOADS; ++c) {
      const int row = (w * C::LOADS + c) * RPL + lane / CPR;
      const int ch = (lane % CPR) ^ sw_xor<RB>(row);
      offd[c] = (uint32_t)(row * D + ch * 8) * 2u;
      offr[c] = (uint32_t)(min(row, N - 1 - kl) * D + ch * 8) * 2u;
    }
  }

  // One key tile, one 32-key block at a time (one S^T / dP^T pair live):
  // S^T = K Q^T and dP^T = V dO^T (one query per lane), the exponent
  // x = S^T*scale*log2e - LSE*log2e, set to -inf for masked keys (a small
  // branch taken only on tiles that cross the diagonal or N; one code path
  // keeps the register allocation within budget), P^T = exp2(x),
  // dS^T = P^T o (dP^T - D) packed per 16-key group t (registers
  // 8*(t&1) .. +7 of the block: k-slot s of half h is key 8*(s/4) + 4h + s%4
  // of the group, the order of the transposing K reads), dQ^T += K^T dS^T.
  // `copy(c)` is called once after each k-step of the first block: the
  // next tile's copies, spread over the MFMA stream. The second block's
  // S^T / dP^T MFMAs come before the first block's dQ^T MFMAs, so that the
  // first block's exp / dS work and the second block's MFMAs (independent of
  // each other) sit together for the scheduler to interleave; every dQ^T
  // accumulator still takes its four MFMAs in the same order (-0.5 to -1.7 %
  // on the backward, bit-identical).
  auto tile = [&](const uint8_t* kt, const uint8_t* vt, int kbase, bool masked, auto&& copy)
                  __attribute__((always_inline)) {
    // S^T and dP^T of 32-key block kb.
    auto sdp = [&](int kb, f32x16& sa, f32x16& pa, bool with_copy) __attribute__((always_inline)) {
      sa = zero16();
      pa = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int o = kb * 32 * RB + rk_off[ks];
        sa = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(kt + o), qreg[ks], sa);
        pa = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(vt + o), doreg[ks], pa);
        if (with_copy) copy(ks);
      }
    };
    // Exponent, mask, P^T, dS^T of block kb, packed per 16-key group.
    auto ds_block = [&](int kb, f32x16& sa, const f32x16& pa, bf16x8 (&sb)[2])
                        __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sa[i] = fmaf(sa[i], c2, nlse2);
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
          sa[i] = (key >= N || (CAUSAL && key > qrow)) ? -INFINITY : sa[i];
        }
      }
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        float ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ds[e] = fast_exp2(sa[8 * th + e]) * (pa[8 * th + e] - drow);
        sb[th] = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      }
    };
    // dQ^T += K^T dS^T for block kb's two 16-key groups.
    auto dq_block = [&](int kb, const bf16x8 (&sb)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        const int t = 2 * kb + th;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dqacc[db] = mfma_32x32x16(tr_operand(kt + 16 * t * RB, tk_off[0][db], tk_off[1][db]),
                                    sb[th], dqacc[db]);
      }
    };
    static_assert(NB == 2, "two 32-key blocks per key tile");
    f32x16 sa, pa;
    bf16x8 sb0[2], sb1[2];
    sdp(0, sa, pa, true);
    ds_block(0, sa, pa, sb0);
    sdp(1, sa, pa, false);
    dq_block(0, sb0);
    ds_block(1, sa, pa, sb1);
    dq_block(1, sb1);
  };

  wait_vmem();
  __syncthreads();
  {
    // Rows 32w .. 32w+31 of the tile: in the first buffer for w < 2.
    const int h = w >> 1;
    const uint8_t* qs = G == 2 ? k_lds[h][1] : (h == 0 ? k_lds[0][1] : v_lds[0][1]);
    const uint8_t* ds = v_lds[h][1];
    const int row = 32 * (w & 1) + l32;
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int o = sw_off<RB>(row, 16 * ks + 8 * hi);
      qreg[ks] = *reinterpret_cast<const bf16x8*>(qs + o);
      if constexpr (G == 2) {
        doreg[ks] = *reinterpret_cast<const bf16x8*>(ds + o);
        oreg[ks] = *reinterpret_cast<const u32x4*>(o_lds + h * C::TILE + o);
      }
      const u32x4 ov = oreg[ks];
      const u32x4 dv = __builtin_bit_cast(u32x4, doreg[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dpart += __uint_as_float(ov[e] << 16) * __uint_as_float(dv[e] << 16);
        dpart += __uint_as_float(ov[e] & 0xffff0000u) * __uint_as_float(dv[e] & 0xffff0000u);
      }
    }
    drow = halves_sum(dpart);
    if (grp == 0 && hi == 0 && qrow < N) Dvec[(size_t)head * N + qrow] = drow;
  }
  // Every wave has its rows before the first step's copies refill the
  // second buffers.
  __syncthreads();

  // Step s: group g computes key tile j = G*s + g and copies its next tile
  // j + G into its other buffers (copy c: K part c/2 for even c, V part c/2
  // for odd c); past the last tile the copies repeat it (in bounds, unused).
  // Every group runs the same number of steps, so all waves meet the same
  // barriers.
  const int ns = (nt + G - 1) / G;
  for (int s = 0; s < ns; ++s) {
    const int b = s & 1;
    const int j = G * s + grp;
    const int kc = min(j + G, nt - 1) * C::BN;
    const bool full = kc + C::BN <= N;
    auto copy = [&](int c) __attribute__((always_inline)) {
      const int i = c >> 1;
      uint8_t* dst = (c & 1) ? v_lds[grp][b ^ 1] : k_lds[grp][b ^ 1];
      const uint16_t* src = ((c & 1) ? V : K) + off + (size_t)kc * D;
      lds_copy16s(src, full ? offd[i] : offr[i], lds_addr(dst + (w * C::LOADS + i) * 1024));
    };
    if (j < ntw) {
      const int kbase = j * C::BN;
      const bool masked = (CAUSAL && kbase + C::BN - 1 > qw) || kbase + C::BN > N;
      tile(k_lds[grp][b], v_lds[grp][b], kbase, masked, copy);
    } else {
#pragma unroll
      for (int c = 0; c < 2 * C::LOADS; ++c) copy(c);
    }
    wait_vmem();
    __syncthreads();
  }

  // ---- The two groups' partial dQ^T are summed through LDS (lane-contiguous
  // fp32, in the K buffers: every read of them finished before the last
  // barrier).
  if constexpr (G == 2) {
    float* red = reinterpret_cast<float*>(k_lds) + w * (DB * 16 * 64) + lane;
    static_assert(4 * DB * 16 * 64 * 4 <= 2 * G * C::TILE, "partial sums fit the K buffers");
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[(db * 16 + i) * 64] = dqacc[db][i];
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) dqacc[db][i] += red[(db * 16 + i) * 64];
  }

  // ---- dQ = scale * dQ^T, out through this wave's slice of group 0's V
  // buffers (free: every step ended with a barrier after its reads and
  // copies, and the group sum above used the K buffers).
  {
    u32x2 qv[DB][4];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        qv[db][g4] = u32x2{pack_bf16x2(dqacc[db][4 * g4 + 0] * scale, dqacc[db][4 * g4 + 1] * scale),
                           pack_bf16x2(dqacc[db][4 * g4 + 2] * scale, dqacc[db][4 * g4 + 3] * scale)};
    store_rows_staged<D>(dQ + off + (size_t)qw * D, N - qw, &v_lds[0][0][0] + w * 32 * RB, qv, lane);
  }
}

// The dQ kernel's key split (two 4-wave groups per 128-query tile taking
// alternate key tiles): causal grids of at most 512 query tiles (one round at
// two workgroups per CU), non-causal grids of at most 256 (one per CU). The
// same rule for both head dimensions.
bool bwd_dq_uses_split(int BH, int N, bool causal) {
  const int ntq = (N + DqCfg<128>::BM - 1) / DqCfg<128>::BM;
  static_assert(DqCfg<128>::BM == DqCfg<64>::BM, "one query-tile size");
  return (int64_t)ntq * BH <= (causal ? 512 : 256);
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const uint16_t* o, const uint16_t* dout, const float* lse,
                             uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dvec, int BH,
                             int N, float scale, hipStream_t stream) {
  const int xcd_group = (BH % 8 == 0) ? BH / 8 : 0;
  {
    // dQ first: it also writes D, which the dK / dV kernel reads.
    using C = DqCfg<D>;
    const int ntq = (N + C::BM - 1) / C::BM;
    dim3 grid((unsigned)(ntq * BH));
    // A causal grid that fits in one round (two 4-wave workgroups per CU on
    // 256 CUs) takes as long as its longest query tile's chain of key tiles:
    // then each tile's key tiles are split over two groups of 4 waves in one
    // workgroup (measured at B=2, H=16, N=2048: -5 us of about 150). So is a
    // non-causal grid of at most one 4-wave workgroup per CU, which would
    // leave one wave per SIMD (backward -5.5 % at B=1, H=8, N=4096 and
    // H=2, N=16384); with two per CU the split is 3 % slower there.
    if (bwd_dq_uses_split(BH, N, CAUSAL))
      hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL, 2>), grid, dim3(2 * C::THREADS), 0,
                         stream, q, k, v, dout, o, lse, dvec, dq, BH, N, ntq, scale * kLog2e,
                         scale, xcd_group);
    else
      hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL, 1>), grid, dim3(C::THREADS), 0, stream,
                         q, k, v, dout, o, lse, dvec, dq, BH, N, ntq, scale * kLog2e, scale,
                         xcd_group);
  }
  {
    using C = BwdCfg<D>;
    const int nkt = (N + C::BNK - 1) / C::BNK;
    const int nunits = CAUSAL ? (nkt + 1) / 2 : nkt;   // causal: key tiles u and nkt-1-u
    dim3 grid((unsigned)(nunits * BH));
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL>), grid, dim3(C::THREADS), 0, stream,
                       q, k, v, dout, lse, dvec, dk, dv, BH, N, nunits, scale * kLog2e, scale,
                       xcd_group);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------- no-allocation scratch
// Device memory for the row statistic D of fa_bwd_noalloc, for callers that
// cannot allocate: a file-scope array that every device holds from the
// library's load until the process ends (16 MiB). In host code the name
// `scratch` is only a host-side handle; its device address is looked up once
// per device with hipGetSymbolAddress and only that address is ever passed to
// a kernel. Nothing in it needs clearing: the dQ kernel writes D for every
// row of the call before the dK/dV kernel, on the same stream, reads it.
constexpr size_t kNoAllocRows = size_t(1) << 22;
static __device__ __align__(256) float scratch[kNoAllocRows];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};
}  // namespace

size_t bwd_noalloc_max_rows() { return kNoAllocRows; }

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept for the life of the process.
hipError_t bwd_noalloc_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

hipError_t bwd_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* o, const uint16_t* dout, const float* lse,
                        uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dvec, int BH, int N,
                        int d, float scale, bool causal, hipStream_t stream) {
#define FA_BWD_CASE(DD, CC) \
  if (d == DD && causal == CC) \
    return launch_bwd<DD, CC>(q, k, v, o, dout, lse, dq, dk, dv, dvec, BH, N, scale, stream);
  FA_BWD_CASE(128, true)
  FA_BWD_CASE(128, false)
  FA_BWD_CASE(64, true)
  FA_BWD_CASE(64, false)
#undef FA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
