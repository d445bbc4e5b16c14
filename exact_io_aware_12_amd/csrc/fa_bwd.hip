// Backward pass of fused exact attention for gfx950.
//
// Method: "FlashAttention core principles" (lesson 1), section 5: only one
// statistic per row is kept from the forward pass; S and P are recomputed tile
// by tile, and per tile pair dV += P^T dO, dP = dO V^T,
// dS = P o (dP - D) (times the scale), dQ += dS K, dK += dS^T Q. The row
// statistic D_i = sum_j P_ij dP_ij is a sum over the WHOLE row (it equals
// dO_i . O_i); taken per tile it would not be the gradient, so it is computed
// once per row before the tile loop.
//
// Three kernels on the caller's stream:
//   1. fa_bwd_pre:   D_i = dO_i . O_i (fp32) and zero the fp32 dQ accumulator.
//   2. fa_bwd_main:  one workgroup per 128-key tile (4 wave64s x 32 keys, one
//      wave per SIMD); the loop runs over 64-query tiles (outer loop over K/V,
//      inner over Q, so dK and dV stay in registers for the whole loop).
//   3. fa_bwd_dq:    dQ = scale * accumulator, rounded to bf16.
//
// gfx950 mapping of the main kernel (32x32x16 bf16 MFMAs, fp32 accumulate):
//   * S = Q K^T and dP = dO V^T are computed with one key per lane (the B
//     operands K and V of this wave's 32 keys live in registers), so P and dS
//     sit in registers in exactly the layout the B operand of
//     dV^T += dO^T P and dK^T += Q^T dS needs (k-slots are queries).
//   * Q and dO tiles go from HBM/L2 straight into LDS (global_load_lds_dwordx4,
//     double-buffered) in one XOR swizzle that serves both the row-major
//     operand reads of S and dP (ds_read_b128) and the transposing reads that
//     give Q^T and dO^T (ds_read_b64_tr_b16) without bank conflicts.
//   * dQ needs dS with one query per lane: dS^T goes to LDS (8-byte writes)
//     and comes back through transposing reads. Each wave owns one 32-wide
//     head-dim block of dQ, so its K operand for dQ += dS K is loaded once
//     into registers; dQ is accumulated in fp32 with hardware float atomics,
//     issued at the start of the next query tile so the per-tile wait only
//     covers copies that had a whole tile's time to land.
//   * Scheduling-group barriers interleave the MFMAs with the VALU work and
//     the LDS operand reads of each phase.
#include "fa_common.h"

namespace fa {

// ----------------------------------------------------------------- kernel 1
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
    float* __restrict__ Dvec, float* __restrict__ dQacc, long long rows) {
  constexpr int TPR = D / 8;            // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;        // rows per block
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + tid / TPR;
  const int c = tid % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = ld_global_16B(O + row * D + c * 8);
    const u32x4 b = ld_global_16B(dO + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += __uint_as_float(a[e] << 16) * __uint_as_float(b[e] << 16);
      acc += __uint_as_float(a[e] & 0xffff0000u) * __uint_as_float(b[e] & 0xffff0000u);
    }
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(dQacc + row * D + c * 8) = z;
    *reinterpret_cast<f32x4*>(dQacc + row * D + c * 8 + 4) = z;
  }
#pragma unroll
  for (int s = TPR / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (row < rows && c == 0) Dvec[row] = acc;
}

// ----------------------------------------------------------------- kernel 3
__global__ __launch_bounds__(256) void fa_bwd_dq_kernel(
    const float* __restrict__ dQacc, uint16_t* __restrict__ dQ, long long n8, float scale) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(dQacc + i * 8);
  const f32x4 b = *reinterpret_cast<const f32x4*>(dQacc + i * 8 + 4);
  u32x4 o = {pack_bf16x2(a[0] * scale, a[1] * scale), pack_bf16x2(a[2] * scale, a[3] * scale),
             pack_bf16x2(b[0] * scale, b[1] * scale), pack_bf16x2(b[2] * scale, b[3] * scale)};
  *reinterpret_cast<u32x4*>(dQ + i * 8) = o;
}

// ----------------------------------------------------------------- kernel 2
#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct BwdCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 256;
  static constexpr int BNK = 128;          // keys per workgroup (32 per wave)
  static constexpr int BMQ = 64;           // queries per inner tile
  static constexpr int RB = D * 2;         // bytes per Q / dO / K row in LDS
  static constexpr int QTILE = BMQ * RB;   // 16 KiB (d=128)
  static constexpr int KTILE = BNK * RB;   // 32 KiB (d=128)
  static constexpr int SRB = BMQ * 2;      // bytes per dS^T row (one key)
  static constexpr int STILE = BNK * SRB;  // 16 KiB
  static constexpr int QLOADS = QTILE / 1024 / WAVES;   // 1 KiB copies per wave
  static constexpr int KLOADS = KTILE / 1024 / WAVES;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int NQB = BMQ / 32;     // 32-query blocks per tile
  static constexpr int DQ_QB = NQB * DB / WAVES;   // dQ query blocks per wave
  static_assert(DQ_QB * WAVES == NQB * DB, "dQ split");
};

// Swizzled byte offset of 2-byte element (row, col) in a tile with R-byte
// rows. Chunks of 16 bytes are XORed with a function of the row that is a
// bijection over 16 consecutive rows (so a row-major operand read of 16 rows
// hits 16 distinct bank groups) and whose top bits follow row%4 (so the 4
// rows of a transposing read fall in 4 distinct 64-byte bank quarters).
template <int R>
__device__ __forceinline__ int sw_off(int row, int col) {
  const int byte = col * 2;
  int f;
  if constexpr (R == 256) f = ((row & 3) << 2) | ((row >> 2) & 3);
  else f = (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  return row * R + ((((byte >> 4) ^ f)) << 4) + (byte & 15);
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
}
__device__ __forceinline__ void lds_copy4(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(lds_addr) : "memory", "m0");
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
    const int pc = lane % CPR;
    int f;
    if constexpr (R == 256) f = ((row & 3) << 2) | ((row >> 2) & 3);
    else f = (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    const int c = pc ^ f;
    const uint16_t* g = src + (size_t)min(row0 + row, N - 1) * D + c * 8;
    lds_copy16(g, lds_addr(lds + lrow * R));
  }
}

// Per-row statistics of one query tile into LDS (64 fp32 LSE, then 64 fp32
// D; rows past N read row N-1): one 4-byte copy per lane of one wave.
__device__ __forceinline__ void dma_stats(const float* __restrict__ lse, const float* __restrict__ dv,
                                          const float* lds, int q0, int N, int lane) {
  lds_copy4(lse + min(q0 + lane, N - 1), lds_addr(lds));
  lds_copy4(dv + min(q0 + lane, N - 1), lds_addr(lds + 64));
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fa_bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dvec,
    float* __restrict__ dQacc, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    int BH, int N, int nunits, float c2, float scale, int xcd_group) {
  using C = BwdCfg<D>;
  constexpr int KS = C::KS, DB = C::DB, NQB = C::NQB, RB = C::RB, SRB = C::SRB;
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[C::KTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds[2][C::QTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t o_lds[2][C::QTILE];   // dO tiles
  __shared__ __attribute__((aligned(1024))) uint8_t s_lds[C::STILE];      // dS^T
  __shared__ __attribute__((aligned(256))) float st_lds[2][2 * C::BMQ];   // LSE, D

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // Workgroup -> (head, work unit). Causal: unit u covers the key tiles u and
  // nkt-1-u: first key tile u with the query tiles in descending order, then
  // key tile nkt-1-u with them in ascending order. Every unit then costs the
  // same number of query-tile steps, and since the units of a head start
  // together, they all work on the same query tile (or two) at any time, so
  // the fp32 dQ rows being accumulated and the Q / dO tiles being read stay
  // in the XCD's L2. Non-causal: one key tile per unit, ascending.
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
  float* dQh = dQacc + off;
  const int nqt = (N + C::BMQ - 1) / C::BMQ;

  // dQ work of this wave: head-dim block dq_db, query blocks dq_qb0.. of each tile.
  const int dq_db = w % DB;
  const int dq_qb0 = (w / DB) * C::DQ_QB;
  // Transposing-read lane offsets: lane (group g = lane/16, source s = lane%16)
  // points at row 4*hi + s/4 (plus 16t + 8*half) and column 16*(g&1) + 4*(s&3)
  // (plus 32*block) of a row-major tile.
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // Per-lane LDS offsets. The swizzles only look at bits 0-3 of the row, so
  // whole 16-row (and 32-row) steps are plain immediate offsets: one register
  // per (half, 32-column block) for transposing reads, one per k-step for
  // the row-major operand reads.
  int tq_off[2][DB];            // Q / dO tiles, transposing reads
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < DB; ++db) tq_off[h][db] = sw_off<RB>(tr_row + 8 * h, 32 * db + tr_col);
  int ts_off[2][C::DQ_QB];      // dS^T tile, transposing reads
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int x = 0; x < C::DQ_QB; ++x)
      ts_off[h][x] = sw_off<SRB>(tr_row + 8 * h, 32 * (dq_qb0 + x) + tr_col);
  int rq_off[KS];               // Q / dO tiles, row-major reads of row l32
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) rq_off[ks] = sw_off<RB>(l32, 16 * ks + 8 * hi);

  bf16x8 kreg[KS], vreg[KS];          // this lane's key row of K and V (B operands)
  bf16x8 ktreg[C::BNK / 16];          // K operand of dQ += dS K (k-slots = keys)
  f32x16 dkacc[DB], dvacc[DB], dqacc[C::DQ_QB];
  int k0 = 0, kk = 0;                 // first key of the tile, this lane's key

  // dQ partial sums of a tile -> fp32 atomics. A full tile takes the
  // branch-free form (uniform base + constant per-lane offsets); only a tile
  // that crosses N needs per-element predicates.
  const int dq_lane = (32 * dq_qb0 + 4 * hi) * D + 32 * dq_db + l32;
  auto flush_dq = [&](int qbase) __attribute__((always_inline)) {
    if (qbase + C::BMQ <= N) {
      float* const base = dQh + (size_t)qbase * D;
#pragma unroll
      for (int x = 0; x < C::DQ_QB; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          unsafeAtomicAdd(base + dq_lane + (32 * x + 8 * (i >> 2) + (i & 3)) * D, dqacc[x][i]);
    } else {
#pragma unroll
      for (int x = 0; x < C::DQ_QB; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = qbase + 32 * (dq_qb0 + x) + 8 * (i >> 2) + 4 * hi + (i & 3);
          if (q < N) unsafeAtomicAdd(dQh + (size_t)q * D + 32 * dq_db + l32, dqacc[x][i]);
        }
    }
  };

  const int nkt_ = (N + C::BNK - 1) / C::BNK;
  const int nparts = (CAUSAL && 2 * unit + 1 != nkt_) ? 2 : 1;
  for (int part = 0; part < nparts; ++part) {
    const int kt = part == 0 ? unit : nkt_ - 1 - unit;
    k0 = kt * C::BNK;
    kk = k0 + 32 * w + l32;
    // Query tiles it_lo .. nqt-1 (causal: from the one holding key k0), in
    // descending order in the first part of a causal unit.
    const bool rev = CAUSAL && part == 0;
    const int it_lo = CAUSAL ? (k0 / C::BMQ) : 0;
    const int nsteps = nqt - it_lo;
    auto tile_at = [&](int step) __attribute__((always_inline)) {
      return rev ? nqt - 1 - step : it_lo + step;
    };

    // Copies: the K tile (for the dQ operands) and the first query tile.
    dma_rows<D, C::KLOADS>(K + off, k_lds, k0, N, w, lane);
    dma_rows<D, C::QLOADS>(Qh, q_lds[0], tile_at(0) * C::BMQ, N, w, lane);
    dma_rows<D, C::QLOADS>(dOh, o_lds[0], tile_at(0) * C::BMQ, N, w, lane);
    if (w == 0) dma_stats(LSEh, Dh, st_lds[0], tile_at(0) * C::BMQ, N, lane);
    {
      const size_t o = (size_t)min(kk, N - 1) * D + hi * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kreg[ks] = __builtin_bit_cast(bf16x8, ld_global_16B(K + off + o + ks * 16));
        vreg[ks] = __builtin_bit_cast(bf16x8, ld_global_16B(V + off + o + ks * 16));
      }
    }
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int t = 0; t < C::BNK / 16; ++t)
      ktreg[t] = tr_operand(k_lds + 16 * t * RB, sw_off<RB>(tr_row, 32 * dq_db + tr_col),
                            sw_off<RB>(tr_row + 8, 32 * dq_db + tr_col));
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      dkacc[i] = zero16();
      dvacc[i] = zero16();
    }

    for (int step = 0; step < nsteps; ++step) {
      // Buffers of this query tile (b) and of the next one (b ^ 1).
      const int b = step & 1;
      const uint8_t* qt = q_lds[b];
      const uint8_t* ot = o_lds[b];
      const float* st = st_lds[b];
      const int qbase = tile_at(step) * C::BMQ;
      if (step + 1 < nsteps) {
        const int qn = tile_at(step + 1) * C::BMQ;
        dma_rows<D, C::QLOADS>(Qh, q_lds[b ^ 1], qn, N, w, lane);
        dma_rows<D, C::QLOADS>(dOh, o_lds[b ^ 1], qn, N, w, lane);
        if (w == 0) dma_stats(LSEh, Dh, st_lds[b ^ 1], qn, N, lane);
      }
      if (step > 0) flush_dq(tile_at(step - 1) * C::BMQ);
      // ---- S = Q K^T and dP = dO V^T (one key per lane, 32 queries per block).
      f32x16 sacc[NQB], pacc[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        sacc[qb] = zero16();
        pacc[qb] = zero16();
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const int o = 32 * qb * RB + rq_off[ks];
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qt + o);
          const bf16x8 ad = *reinterpret_cast<const bf16x8*>(ot + o);
          sacc[qb] = mfma_32x32x16(aq, kreg[ks], sacc[qb]);
          pacc[qb] = mfma_32x32x16(ad, vreg[ks], pacc[qb]);
        }
      // ---- P = exp2(S*scale*log2e - LSE*log2e), dS = P o (dP - D), packed to
      // bf16 right away (k-slot order of the dV / dK B operands: 16 queries per
      // step t, registers 8*(t&1) .. +7 of block t/2).
      const bool masked = (CAUSAL && qbase < k0 + C::BNK - 1) || qbase + C::BMQ > N ||
                          k0 + C::BNK > N;
      bf16x8 pbv[C::BMQ / 16], sbv[C::BMQ / 16];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float pv[8], dv8[8];
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            const int g4 = 2 * half + g2;
            const int ql = 32 * qb + 8 * g4 + 4 * hi;     // first of 4 consecutive queries
            const f32x4 lse4 = *reinterpret_cast<const f32x4*>(st + ql);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(st + C::BMQ + ql);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * g4 + e;
              float p = fast_exp2(fmaf(sacc[qb][i], c2, -lse4[e] * kLog2e));
              if (masked) {
                const int q = qbase + ql + e;
                if ((CAUSAL && kk > q) || kk >= N || q >= N) p = 0.f;
              }
              pv[4 * g2 + e] = p;
              dv8[4 * g2 + e] = p * (pacc[qb][i] - d4[e]);
            }
          }
          const int t = 2 * qb + half;
          pbv[t] = pack_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
          sbv[t] = pack_bf16x8(dv8[0], dv8[1], dv8[2], dv8[3], dv8[4], dv8[5], dv8[6], dv8[7]);
        }
      // ---- dV^T += dO^T P and dK^T += Q^T dS (k-slots = queries).
#pragma unroll
      for (int t = 0; t < C::BMQ / 16; ++t) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dvacc[db] = mfma_32x32x16(tr_operand(ot + 16 * t * RB, tq_off[0][db], tq_off[1][db]), pbv[t], dvacc[db]);
          dkacc[db] = mfma_32x32x16(tr_operand(qt + 16 * t * RB, tq_off[0][db], tq_off[1][db]), sbv[t], dkacc[db]);
        }
      }
      // ---- dS^T (bf16) to LDS: row = this lane's key, 4 consecutive queries
      // (one half of a packed operand) per write.
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const u32x4 w4 = __builtin_bit_cast(u32x4, sbv[2 * qb + (g4 >> 1)]);
          const u32x2 v = {w4[2 * (g4 & 1)], w4[2 * (g4 & 1) + 1]};
          *reinterpret_cast<u32x2*>(s_lds + sw_off<SRB>(32 * w + l32, 32 * qb + 8 * g4 + 4 * hi)) = v;
        }
      {
        constexpr int kMfma = 0x008, kValu = 0x002, kDsRead = 0x100;
        // S / dP MFMAs each with one operand read; the dV / dK MFMAs each with
        // two transposing reads and the exp / dS / packing work.
        __builtin_amdgcn_sched_group_barrier(kDsRead, 4, 0);
#pragma unroll
        for (int i = 0; i < 2 * KS * NQB; ++i) {
          __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 2 * (C::BMQ / 16) * DB; ++i) {
          __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
          __builtin_amdgcn_sched_group_barrier(kValu, 6, 0);
        }
      }
      __syncthreads();
      // ---- dQ (this wave's head-dim block) = dS K over the 128 keys.
#pragma unroll
      for (int x = 0; x < C::DQ_QB; ++x) {
        dqacc[x] = zero16();
#pragma unroll
        for (int t = 0; t < C::BNK / 16; ++t) {
          const bf16x8 a = tr_operand(s_lds + 16 * t * SRB, ts_off[0][x], ts_off[1][x]);
          dqacc[x] = mfma_32x32x16(a, ktreg[t], dqacc[x]);
        }
      }
      wait_vmem();
      __syncthreads();
    }
    flush_dq(tile_at(nsteps - 1) * C::BMQ);

    // ---- dK = scale * dK^T, dV = dV^T (one key per lane; 4 consecutive d).
    if (kk < N) {
      uint16_t* dkrow = dK + off + (size_t)kk * D;
      uint16_t* dvrow = dV + off + (size_t)kk * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * hi;
          const f32x16& a = dkacc[db];
          const f32x16& b = dvacc[db];
          u32x2 pk = {pack_bf16x2(a[4 * g4] * scale, a[4 * g4 + 1] * scale),
                      pack_bf16x2(a[4 * g4 + 2] * scale, a[4 * g4 + 3] * scale)};
          u32x2 pv = {pack_bf16x2(b[4 * g4], b[4 * g4 + 1]),
                      pack_bf16x2(b[4 * g4 + 2], b[4 * g4 + 3])};
          *reinterpret_cast<u32x2*>(dkrow + d0) = pk;
          *reinterpret_cast<u32x2*>(dvrow + d0) = pv;
        }
    }
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const uint16_t* o, const uint16_t* dout, const float* lse,
                             uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dqacc,
                             float* dvec, int BH, int N, float scale, hipStream_t stream) {
  using C = BwdCfg<D>;
  const long long rows = (long long)BH * N;
  {
    constexpr int RPB = 256 / (D / 8);
    dim3 grid((unsigned)((rows + RPB - 1) / RPB));
    hipLaunchKernelGGL((fa_bwd_pre_kernel<D>), grid, dim3(256), 0, stream, o, dout, dvec,
                       dqacc, rows);
  }
  {
    const int nkt = (N + C::BNK - 1) / C::BNK;
    const int nunits = CAUSAL ? (nkt + 1) / 2 : nkt;   // causal: key tiles u and nkt-1-u
    const int xcd_group = (BH % 8 == 0) ? BH / 8 : 0;
    dim3 grid((unsigned)(nunits * BH));
    hipLaunchKernelGGL((fa_bwd_main_kernel<D, CAUSAL>), grid, dim3(C::THREADS), 0, stream,
                       q, k, v, dout, lse, dvec, dqacc, dk, dv, BH, N, nunits, scale * kLog2e,
                       scale, xcd_group);
  }
  {
    const long long n8 = rows * D / 8;
    dim3 grid((unsigned)((n8 + 255) / 256));
    hipLaunchKernelGGL(fa_bwd_dq_kernel, grid, dim3(256), 0, stream, dqacc, dq, n8, scale);
  }
  return hipGetLastError();
}

hipError_t bwd_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* o, const uint16_t* dout, const float* lse,
                        uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dqacc, float* dvec,
                        int BH, int N, int d, float scale, bool causal, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_bwd<128, true>(q, k, v, o, dout, lse, dq, dk, dv, dqacc, dvec, BH,
                                          N, scale, stream)
                  : launch_bwd<128, false>(q, k, v, o, dout, lse, dq, dk, dv, dqacc, dvec, BH,
                                           N, scale, stream);
  return causal ? launch_bwd<64, true>(q, k, v, o, dout, lse, dq, dk, dv, dqacc, dvec, BH, N,
                                       scale, stream)
                : launch_bwd<64, false>(q, k, v, o, dout, lse, dq, dk, dv, dqacc, dvec, BH, N,
                                        scale, stream);
}

}  // namespace fa
