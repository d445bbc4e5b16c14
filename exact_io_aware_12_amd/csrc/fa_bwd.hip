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
//   2. fa_bwd_main:  one workgroup per 128-key tile (4 wave64s x 32 keys); the
//      loop runs over 64-query tiles (outer loop over K/V, inner over Q, so
//      dK and dV stay in registers for the whole loop).
//   3. fa_bwd_dq:    dQ = scale * accumulator, rounded to bf16.
//
// gfx950 mapping of the main kernel (32x32x16 bf16 MFMAs, fp32 accumulate):
//   * S = Q K^T and dP = dO V^T are computed with one key per lane (the B
//     operands K and V of this wave's 32 keys live in registers), so P and dS
//     sit in registers in exactly the layout the B operand of
//     dV^T += dO^T P and dK^T += Q^T dS needs (k-slots are queries).
//   * Q and dO tiles are stored in LDS twice: row-major (A operands of S and
//     dP) and transposed with queries permuted inside groups of 16 to match
//     the accumulator's row order (A operands of dV^T and dK^T).
//   * dQ needs dS with one query per lane, so dS goes through LDS (bf16) and
//     dQ += dS K is accumulated in fp32 with hardware float atomics.
//   * The next Q/dO tile is prefetched into registers during the compute;
//     two barriers per tile.
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
template <int D>
struct BwdCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 256;
  static constexpr int BNK = 128;          // keys per workgroup (32 per wave)
  static constexpr int BMQ = 64;           // queries per inner tile
  static constexpr int QS = D + 8;         // row-major Q / dO stride (bf16)
  static constexpr int TS = BMQ + 8;       // transposed Q / dO stride
  static constexpr int SS = BNK + 8;       // dS stride
  static constexpr int KTS = BNK + 8;      // K^T stride
  static constexpr int KCH = D / 8;        // 16-byte chunks per row
  static constexpr int UNITS = (BMQ / 4) * KCH;   // 4-row x 16-byte load units
  static constexpr int DB = D / 32;
  static constexpr int NQB = BMQ / 32;     // 32-query blocks per tile
  static constexpr int DQ_BLOCKS = NQB * DB;      // 32x32 dQ blocks per tile
  static constexpr int DQ_PER_WAVE = DQ_BLOCKS / WAVES;
  static_assert(UNITS <= THREADS, "one load unit per thread at most");
  static_assert(DQ_PER_WAVE * WAVES == DQ_BLOCKS, "dQ split");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fa_bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dvec,
    float* __restrict__ dQacc, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    int BH, int N, int nkt, float c2, float scale, int xcd_group) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[C::BMQ * C::QS];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[C::BMQ * C::QS];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * C::TS];
  __shared__ __attribute__((aligned(16))) uint16_t dOt[D * C::TS];
  __shared__ __attribute__((aligned(16))) uint16_t dSs[C::BMQ * C::SS];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * C::KTS];
  __shared__ float lse2s[C::BMQ];
  __shared__ float Ds[C::BMQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
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
  // Causal: key tile 0 sees every query, the last one the fewest; issue the
  // heaviest first.
  const int kt = rank;
  const int k0 = kt * C::BNK;
  const int kk = k0 + 32 * w + l32;        // this lane's key
  const size_t off = (size_t)head * N * D;
  const uint16_t* Qh = Q + off;
  const uint16_t* dOh = dO + off;
  const float* LSEh = LSE + (size_t)head * N;
  const float* Dh = Dvec + (size_t)head * N;
  float* dQh = dQacc + off;

  // This lane's key row of K and V as B operands (k-slots = head dim).
  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const size_t o = (size_t)kk * D + ks * 16 + hi * 8;
    u32x4 a = kk < N ? ld_global_16B(K + off + o) : zero_u32x4();
    u32x4 b = kk < N ? ld_global_16B(V + off + o) : zero_u32x4();
    kreg[ks] = __builtin_bit_cast(bf16x8, a);
    vreg[ks] = __builtin_bit_cast(bf16x8, b);
  }
  // K^T of the whole key tile in LDS (B operand of dQ += dS K).
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const u32x4 a = __builtin_bit_cast(u32x4, kreg[ks]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t word = a[e >> 1];
      const uint16_t h = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xffffu);
      Kt[(ks * 16 + hi * 8 + e) * C::KTS + 32 * w + l32] = h;
    }
  }

  f32x16 dkacc[C::DB], dvacc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) {
    dkacc[i] = zero16();
    dvacc[i] = zero16();
  }

  const int nqt = (N + C::BMQ - 1) / C::BMQ;
  const int it0 = CAUSAL ? (k0 / C::BMQ) : 0;

  u32x4 qld[4], dld[4];
  float lse_ld = 0.f, d_ld = 0.f;
  const bool loader = tid < C::UNITS;
  const int ucc = tid % C::KCH, ug = tid / C::KCH;   // chunk, 4-row group

  auto load_tile = [&](int it) {
    const int qb0 = it * C::BMQ;
    if (loader) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int q = qb0 + 4 * ug + b;
        qld[b] = q < N ? ld_global_16B(Qh + (size_t)q * D + ucc * 8) : zero_u32x4();
        dld[b] = q < N ? ld_global_16B(dOh + (size_t)q * D + ucc * 8) : zero_u32x4();
      }
    }
    if (tid < C::BMQ) {
      const int q = qb0 + tid;
      lse_ld = q < N ? LSEh[q] * kLog2e : INFINITY;   // P = 0 for padded rows
      d_ld = q < N ? Dh[q] : 0.f;
    }
  };
  auto store_tile = [&]() {
    if (loader) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = 4 * ug + b;
        *reinterpret_cast<u32x4*>(Qs + r * C::QS + ucc * 8) = qld[b];
        *reinterpret_cast<u32x4*>(dOs + r * C::QS + ucc * 8) = dld[b];
      }
      // Rows 4g..4g+3 (g = 4t + 2a + h) -> transposed positions 16t + 8h + 4a.
      const int pos = 16 * (ug >> 2) + 8 * (ug & 1) + 4 * ((ug >> 1) & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dw = e >> 1;
        u32x2 pq, pd;
        if (e & 1) {
          pq = u32x2{pack_hi16(qld[0][dw], qld[1][dw]), pack_hi16(qld[2][dw], qld[3][dw])};
          pd = u32x2{pack_hi16(dld[0][dw], dld[1][dw]), pack_hi16(dld[2][dw], dld[3][dw])};
        } else {
          pq = u32x2{pack_lo16(qld[0][dw], qld[1][dw]), pack_lo16(qld[2][dw], qld[3][dw])};
          pd = u32x2{pack_lo16(dld[0][dw], dld[1][dw]), pack_lo16(dld[2][dw], dld[3][dw])};
        }
        *reinterpret_cast<u32x2*>(Qt + (ucc * 8 + e) * C::TS + pos) = pq;
        *reinterpret_cast<u32x2*>(dOt + (ucc * 8 + e) * C::TS + pos) = pd;
      }
    }
    if (tid < C::BMQ) {
      lse2s[tid] = lse_ld;
      Ds[tid] = d_ld;
    }
  };

  if (it0 < nqt) {
    load_tile(it0);
    store_tile();
  }

  for (int it = it0; it < nqt; ++it) {
    __syncthreads();
    if (it + 1 < nqt) load_tile(it + 1);
    const int qbase = it * C::BMQ;

    // ---- S = Q K^T and dP = dO V^T (one key per lane).
    f32x16 sacc[C::NQB], pacc[C::NQB];
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      sacc[qb] = zero16();
      pacc[qb] = zero16();
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int o = (qb * 32 + l32) * C::QS + ks * 16 + hi * 8;
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qs + o);
        const bf16x8 ad = *reinterpret_cast<const bf16x8*>(dOs + o);
        sacc[qb] = mfma_32x32x16(aq, kreg[ks], sacc[qb]);
        pacc[qb] = mfma_32x32x16(ad, vreg[ks], pacc[qb]);
      }
    }
    // ---- P = exp(S*scale - LSE) (base 2), dS = P o (dP - D).
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = qb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
        const int q = qbase + qi;
        float p = fast_exp2(fmaf(sacc[qb][i], c2, -lse2s[qi]));
        if ((CAUSAL && kk > q) || kk >= N) p = 0.f;
        sacc[qb][i] = p;
        pacc[qb][i] = p * (pacc[qb][i] - Ds[qi]);
      }
    // ---- dV^T += dO^T P and dK^T += Q^T dS (k-slots = queries).
#pragma unroll
    for (int t = 0; t < C::BMQ / 16; ++t) {
      const int r0 = (t & 1) * 8;
      const f32x16& p = sacc[t >> 1];
      const f32x16& s = pacc[t >> 1];
      const bf16x8 pb = pack_bf16x8(p[r0], p[r0 + 1], p[r0 + 2], p[r0 + 3], p[r0 + 4],
                                    p[r0 + 5], p[r0 + 6], p[r0 + 7]);
      const bf16x8 sb = pack_bf16x8(s[r0], s[r0 + 1], s[r0 + 2], s[r0 + 3], s[r0 + 4],
                                    s[r0 + 5], s[r0 + 6], s[r0 + 7]);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int o = (db * 32 + l32) * C::TS + 16 * t + 8 * hi;
        const bf16x8 ad = *reinterpret_cast<const bf16x8*>(dOt + o);
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qt + o);
        dvacc[db] = mfma_32x32x16(ad, pb, dvacc[db]);
        dkacc[db] = mfma_32x32x16(aq, sb, dkacc[db]);
      }
    }
    // ---- dS (bf16) to LDS, one query per row.
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int qi = qb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
        const uint32_t pr = pack_bf16x2(pacc[qb][i], pacc[qb][i + 1]);
        dSs[qi * C::SS + 32 * w + l32] = (uint16_t)(pr & 0xffffu);
        dSs[(qi + 1) * C::SS + 32 * w + l32] = (uint16_t)(pr >> 16);
      }
    __syncthreads();
    // ---- dQ += dS K over the 128 keys of this workgroup (fp32 atomics).
#pragma unroll
    for (int x = 0; x < C::DQ_PER_WAVE; ++x) {
      const int bi = w + C::WAVES * x;
      const int qb = bi % C::NQB, db = bi / C::NQB;
      f32x16 acc = zero16();
#pragma unroll
      for (int t = 0; t < C::BNK / 16; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            dSs + (qb * 32 + l32) * C::SS + 16 * t + 8 * hi);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(
            Kt + (db * 32 + l32) * C::KTS + 16 * t + 8 * hi);
        acc = mfma_32x32x16(a, b, acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = qbase + qb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
        if (q < N) unsafeAtomicAdd(dQh + (size_t)q * D + db * 32 + l32, acc[i]);
      }
    }
    if (it + 1 < nqt) store_tile();
  }

  // ---- dK = scale * dK^T, dV = dV^T (one key per lane; 4 consecutive d).
  if (kk < N) {
    uint16_t* dkrow = dK + off + (size_t)kk * D;
    uint16_t* dvrow = dV + off + (size_t)kk * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
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
    const int xcd_group = (BH % 8 == 0) ? BH / 8 : 0;
    dim3 grid((unsigned)(nkt * BH));
    hipLaunchKernelGGL((fa_bwd_main_kernel<D, CAUSAL>), grid, dim3(C::THREADS), 0, stream,
                       q, k, v, dout, lse, dvec, dqacc, dk, dv, BH, N, nkt, scale * kLog2e,
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
