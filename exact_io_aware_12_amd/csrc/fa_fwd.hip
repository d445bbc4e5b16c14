// Forward pass of fused exact attention for gfx950.
//
// Method: "FlashAttention core principles" (lesson 1), sections 3-4: the outer
// loop runs over query tiles (one workgroup per tile), the inner loop streams
// key/value tiles through on-chip memory, keeps a running row max m and row
// sum l, rescales the partial output by exp(m_old - m_new) when the max grows,
// and normalises once at the end. The single-exponential update of the
// interview answer ("2. Online Softmax") and of "FlashAttention and Triton",
// section 19.12 is used: p = exp(s - m_new), l = alpha*l + rowsum(p).
//
// gfx950 mapping
//   * Workgroup = 4 wave64s = BM = 128 query rows; each wave owns 32 rows.
//   * Scores are computed transposed, S^T = K Q^T, with 32x32x16 bf16 MFMAs:
//     the accumulator puts one query per lane (column) and 16 keys per lane
//     (rows), so the row max / row sum are in-lane reductions plus a single
//     exchange between the two 32-lane halves.
//   * O^T = V^T P^T, again one query per lane: P^T goes from the score
//     accumulator into the B operand by register conversion only (bf16), and
//     the per-row rescale alpha is a per-lane scalar.
//   * Q stays in registers for the whole key loop (B operand of S^T).
//   * K tiles sit row-major in LDS (A operand of S^T, one 16-byte read per
//     lane per MFMA). V tiles are transposed while being written to LDS, with
//     keys permuted inside each group of 16 to match the accumulator's row
//     order, so each V^T operand is one 16-byte LDS read as well.
//   * Register-staged double buffering: the global loads of tile j+1 are in
//     flight while tile j is computed from LDS; one barrier per tile.
//   * Softmax runs in the base-2 domain: scores are multiplied by
//     scale*log2(e) in fp32 (Q is never pre-scaled in bf16) and exponentials
//     use v_exp_f32. LSE is converted back to natural log on store.
//   * Causal: tiles above the diagonal are never loaded or computed; only
//     tiles that cross the diagonal (or the ragged end) evaluate the mask.
//     Query tiles are issued heaviest first, and workgroups of one head are
//     kept on one XCD (consecutive workgroup ids go to different XCDs).
#include "fa_common.h"

namespace fa {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;              // query rows per workgroup
  static constexpr int WAVES = 4;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int BN = 8192 / D;         // keys per tile (16 KiB of K)
  static constexpr int KS = D + 8;            // LDS row stride of K (bf16)
  static constexpr int VS = BN + 8;           // LDS row stride of V^T (bf16)
  static constexpr int KBUF = BN * KS;        // elements per K buffer
  static constexpr int VBUF = D * VS;         // elements per V^T buffer
  static constexpr int KCH = D / 8;           // 16-byte chunks per row
  static constexpr int KLD = BN * KCH / THREADS;        // K chunks per thread
  static constexpr int VLD = (BN / 4) * KCH / THREADS;  // V 4-row units per thread
  static constexpr int NB = BN / 32;          // 32-key score blocks per tile
  static constexpr int DB = D / 32;           // 32-wide output blocks
  static constexpr int LDS_BYTES = 2 * (KBUF + VBUF) * 2;
  static_assert(KLD * THREADS == BN * KCH, "K tile split");
  static_assert(VLD * THREADS == (BN / 4) * KCH, "V tile split");
};

// Slack (log2 units) before the running max is moved; see the kernel.
constexpr float kRescaleSlack = 8.f;

// Max / min / sum over the NB*16 score registers of a lane (tree order, so
// the compiler can use 3-input max and independent adds).
template <int NB>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[NB]) {
  float r[NB * 4];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      r[kb * 4 + g] = fmaxf(fmaxf(s[kb][4 * g], s[kb][4 * g + 1]),
                            fmaxf(s[kb][4 * g + 2], s[kb][4 * g + 3]));
#pragma unroll
  for (int w = NB * 4; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) r[i] = fmaxf(r[i], r[i + w / 2]);
  return r[0];
}
template <int NB>
__device__ __forceinline__ float tile_min(const f32x16 (&s)[NB]) {
  float r[NB * 4];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      r[kb * 4 + g] = fminf(fminf(s[kb][4 * g], s[kb][4 * g + 1]),
                            fminf(s[kb][4 * g + 2], s[kb][4 * g + 3]));
#pragma unroll
  for (int w = NB * 4; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) r[i] = fminf(r[i], r[i + w / 2]);
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

// Two workgroups (8 waves) per CU: one wave's softmax runs while the other
// wave on the same SIMD issues MFMAs, which a single wave cannot overlap.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int BH, int N, int ntq, float c2, int xcd_group) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (C::KBUF + C::VBUF)];
  uint16_t* Ks = smem;                      // [2][BN][KS]
  uint16_t* Vt = smem + 2 * C::KBUF;        // [2][D][VS]

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // Workgroup -> (head, query tile).
  int head, rank;
  {
    const int b = blockIdx.x;
    if (xcd_group > 0) {
      // Workgroups are dispatched round-robin over the 8 XCDs; give XCD x the
      // heads [x*G, (x+1)*G) so their K/V stay in that XCD's L2.
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
  const int qw = q0 + w * 32;          // first query row of this wave
  const int qrow = qw + l32;           // this lane's query row
  const size_t off = (size_t)head * N * D;
  const uint16_t* Qh = Q + off;
  const uint16_t* Kh = K + off;
  const uint16_t* Vh = V + off;

  // Q rows of this lane as B operands (k-slots = head-dim positions).
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 t = qrow < N ? ld_global_16B(Qh + (size_t)qrow * D + ks * 16 + hi * 8) : zero_u32x4();
    qreg[ks] = __builtin_bit_cast(bf16x8, t);
  }

  const int kend = CAUSAL ? min(N, q0 + C::BM) : N;
  const int nt = (kend + C::BN - 1) / C::BN;

  u32x4 kreg[C::KLD];
  u32x4 vreg[C::VLD][4];

  auto load_tile = [&](int j) {
    const int kb0 = j * C::BN;
#pragma unroll
    for (int i = 0; i < C::KLD; ++i) {
      const int u = tid + i * C::THREADS;
      const int r = u / C::KCH, cc = u % C::KCH;
      const int key = kb0 + r;
      kreg[i] = key < N ? ld_global_16B(Kh + (size_t)key * D + cc * 8) : zero_u32x4();
    }
#pragma unroll
    for (int i = 0; i < C::VLD; ++i) {
      const int u = tid + i * C::THREADS;
      const int g = u % (C::BN / 4), cc = u / (C::BN / 4);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int key = kb0 + 4 * g + b;
        vreg[i][b] = key < N ? ld_global_16B(Vh + (size_t)key * D + cc * 8) : zero_u32x4();
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* kd = Ks + buf * C::KBUF;
    uint16_t* vd = Vt + buf * C::VBUF;
#pragma unroll
    for (int i = 0; i < C::KLD; ++i) {
      const int u = tid + i * C::THREADS;
      const int r = u / C::KCH, cc = u % C::KCH;
      *reinterpret_cast<u32x4*>(kd + r * C::KS + cc * 8) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::VLD; ++i) {
      // Consecutive lanes take consecutive 4-key groups of one 8-column
      // chunk, so each transposed store instruction writes whole V^T rows
      // (no LDS bank conflicts).
      const int u = tid + i * C::THREADS;
      const int g = u % (C::BN / 4), cc = u / (C::BN / 4);
      // Keys 4g..4g+3: g = 4t + 2a + h lands at positions 16t + 8h + 4a + 0..3.
      const int pos = 16 * (g >> 2) + 8 * (g & 1) + 4 * ((g >> 1) & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dw = e >> 1;
        uint32_t w0, w1;
        if (e & 1) {
          w0 = pack_hi16(vreg[i][0][dw], vreg[i][1][dw]);
          w1 = pack_hi16(vreg[i][2][dw], vreg[i][3][dw]);
        } else {
          w0 = pack_lo16(vreg[i][0][dw], vreg[i][1][dw]);
          w1 = pack_lo16(vreg[i][2][dw], vreg[i][3][dw]);
        }
        u32x2 pr = {w0, w1};
        *reinterpret_cast<u32x2*>(vd + (cc * 8 + e) * C::VS + pos) = pr;
      }
    }
  };

  f32x16 oacc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;   // running max of this lane's row (log2 domain)
  float l_run = 0.f;         // running sum over this lane's half of the keys

  load_tile(0);
  store_tile(0);

  for (int j = 0; j < nt; ++j) {
    __syncthreads();
    if (j + 1 < nt) load_tile(j + 1);
    const int buf = j & 1;
    const int kbase = j * C::BN;
    const bool active = !CAUSAL || kbase <= qw + 31;
    if (active) {
      const uint16_t* kd = Ks + buf * C::KBUF;
      const uint16_t* vd = Vt + buf * C::VBUF;
      // ---- S^T = K Q^T for this tile (NB blocks of 32 keys x 32 queries).
      f32x16 sacc[C::NB];
#pragma unroll
      for (int kb = 0; kb < C::NB; ++kb) {
        sacc[kb] = zero16();
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              kd + (kb * 32 + l32) * C::KS + ks * 16 + hi * 8);
          sacc[kb] = mfma_32x32x16(a, qreg[ks], sacc[kb]);
        }
      }
      // ---- online softmax statistics (base 2).
      // The running max is only moved when a row's tile max exceeds it by
      // more than kRescaleSlack (log2 units); otherwise the stale max is
      // kept, so exp2(s - m) <= 2^kRescaleSlack and the rescale of O and l
      // (64 multiplies per lane) is skipped. The result is unchanged: l and
      // O are both taken relative to the same m, and LSE = m + log2(l).
      const bool need_mask = (CAUSAL && kbase + C::BN - 1 > qw) || (kbase + C::BN > N);
      float tmax;
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kbase + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
            const bool ok = key < N && (!CAUSAL || key <= qrow);
            sacc[kb][i] = ok ? sacc[kb][i] * c2 : -INFINITY;
          }
        tmax = tile_max<C::NB>(sacc);
      } else if (c2 >= 0.f) {
        tmax = tile_max<C::NB>(sacc) * c2;
      } else {
        tmax = tile_min<C::NB>(sacc) * c2;
      }
      tmax = fmaxf(tmax, swap_halves(tmax));
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
      // Rows with no admissible key so far keep m = -inf; their scores are
      // all -inf, so subtracting 0 gives p = 0.
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[kb][i] = fast_exp2(sacc[kb][i] - m_use);
      } else {
        const float nm = -m_use;
#pragma unroll
        for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[kb][i] = fast_exp2(fmaf(sacc[kb][i], c2, nm));
      }
      l_run += tile_sum<C::NB>(sacc);
      // ---- O^T += V^T P^T: 16 keys per MFMA; P^T straight from the
      // accumulator registers (k-slot s of half h = key 8*(s/4) + 4h + s%4).
#pragma unroll
      for (int t = 0; t < C::BN / 16; ++t) {
        const f32x16& p = sacc[t >> 1];
        const int r0 = (t & 1) * 8;
        const bf16x8 pb = pack_bf16x8(p[r0 + 0], p[r0 + 1], p[r0 + 2], p[r0 + 3],
                                      p[r0 + 4], p[r0 + 5], p[r0 + 6], p[r0 + 7]);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              vd + (db * 32 + l32) * C::VS + 16 * t + 8 * hi);
          oacc[db] = mfma_32x32x16(a, pb, oacc[db]);
        }
      }
    }
    if (j + 1 < nt) store_tile((j + 1) & 1);
  }

  // ---- epilogue: O = O / l, LSE = ln2 * (m + log2 l).
  const float l_tot = l_run + swap_halves(l_run);
  if (qrow < N) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = O + off + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hi;
        u32x2 pr = {pack_bf16x2(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv),
                    pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = pr;
      }
    if (hi == 0) LSE[(size_t)head * N + qrow] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint16_t* o, float* lse, int BH, int N, float scale,
                             hipStream_t stream) {
  using C = FwdCfg<D>;
  const int ntq = (N + C::BM - 1) / C::BM;
  const int xcd_group = (BH % 8 == 0) ? BH / 8 : 0;
  const float c2 = scale * kLog2e;
  dim3 grid((unsigned)(ntq * BH)), block(C::THREADS);
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL>), grid, block, 0, stream,
                     q, k, v, o, lse, BH, N, ntq, c2, xcd_group);
  return hipGetLastError();
}

hipError_t fwd_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        uint16_t* o, float* lse, int BH, int N, int d, float scale,
                        bool causal, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_fwd<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch_fwd<128, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch_fwd<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch_fwd<64, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace fa
