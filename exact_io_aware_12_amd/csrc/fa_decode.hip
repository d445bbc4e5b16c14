// Decode attention for gfx950: a few query rows (Nq <= 32) against a long
// key/value cache (Nk rows), e.g. one generated token per sequence.
//
// Method: the same exact attention and online softmax as the forward pass
// ("FlashAttention core principles", lesson 1, sections 3-4), applied to a
// rectangular S; the interview answer's bonus points name this use
// (inference with a KV cache). With so few queries the work is bound by
// reading K and V from HBM, so the key range is split over many workgroups
// (split-K), each producing a partial (O, LSE) over its keys, and a second
// kernel merges the partials with the online-softmax rescaling of lesson 1,
// section 3: LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
//
// gfx950 mapping (one wave64 per workgroup, two waves per SIMD):
//   * S^T = K Q^T with 32x32x16 bf16 MFMAs: one query per lane column (the
//     queries, padded to 32, are the B operand, loaded once), 32 keys per
//     step. K rows go from HBM straight into registers as the A operand.
//   * O^T += V^T P^T: P^T goes from the score accumulator into the B operand
//     by register conversion only; V tiles go HBM -> LDS (global_load_lds,
//     double-buffered, XOR-swizzled) and V^T comes from transposing LDS reads.
//   * The next step's K loads and V copy are issued before the current
//     step's MFMAs; with eight such waves per CU there are ~128 KiB of reads
//     in flight per CU.
#include "fa_common.h"

namespace fa {

#define LDS_AS __attribute__((address_space(3)))

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct DecCfg {
  static constexpr int BK = 32;                 // keys per step
  static constexpr int RB = D * 2;              // bytes per V row in LDS
  static constexpr int TILE = BK * RB;          // 8 KiB (d=128)
  static constexpr int LOADS = TILE / 1024;     // 1 KiB copies per step
  static constexpr int ROWS_PER_LOAD = 1024 / RB;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
};

// Byte offset of (row, column col) of a V tile in LDS: 64-byte blocks are
// XOR-swizzled so the 4 rows of one transposing read hit distinct banks.
template <int D>
__device__ __forceinline__ int dv_off(int row, int col) {
  const int blk = col >> 5, in = (col & 31) * 2;
  if constexpr (D == 128) return row * 256 + ((blk ^ (row & 3)) << 6) + in;
  else return row * 128 + ((blk ^ ((row >> 1) & 1)) << 6) + in;
}

// Element offset (row * D + column) that lane `lane` of copy c fetches: lane
// l writes physical 16-byte chunk l % (RB/16) of row c*ROWS_PER_LOAD +
// l / (RB/16), so it reads the logical chunk the swizzle puts there.
template <int D>
__device__ __forceinline__ int dv_src(int c, int lane, int& row) {
  using C = DecCfg<D>;
  row = c * C::ROWS_PER_LOAD + lane / (C::RB / 16);
  const int pc = lane % (C::RB / 16);
  int lb;
  if constexpr (D == 128) lb = (pc >> 2) ^ (row & 3);
  else lb = (pc >> 2) ^ ((row >> 1) & 1);
  return row * D + lb * 32 + (pc & 3) * 8;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// global_load_lds_dwordx4 in the scalar-base form (lane i writes LDS bytes
// [M0 + 16i, +16)); M0 is written here, hence the clobber and the pragma.
__device__ __forceinline__ void dcopy16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
  strict_copy_wait();
}
#pragma clang diagnostic pop

// Partial attention of all Nq queries over the keys of one split.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_decode_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ Opart, float* __restrict__ Lpart,
    int Nq, int Nk, int nsplit, int chunk, float c2) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[2][C::TILE];
  const int lane = threadIdx.x;
  const int l32 = lane & 31, hi = lane >> 5;
  const int bh = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
  const int k_lo = sp * chunk;
  const int k_hi = min(Nk, k_lo + chunk);
  const int nt = (k_hi - k_lo + C::BK - 1) / C::BK;
  const uint16_t* Kh = K + (size_t)bh * Nk * D;
  const uint16_t* Vh = V + (size_t)bh * Nk * D;
  const int q = l32;                         // this lane's query (column)
  const int qc = min(q, Nq - 1);             // rows past Nq compute with row Nq-1
  const int qpos = Nk - Nq + q;              // its position (causal: last Nq keys)

  // Per-lane offsets of this lane's V copies for a full tile and for the
  // globally last tile when it is ragged (rows past Nk read row Nk-1).
  uint32_t offd[C::LOADS], offr[C::LOADS];
  {
    const int kl = (Nk - 1) / C::BK * C::BK;
#pragma unroll
    for (int c = 0; c < C::LOADS; ++c) {
      int row;
      const int e = dv_src<D>(c, lane, row);
      offd[c] = (uint32_t)e * 2u;
      offr[c] = (uint32_t)(e + (min(row, Nk - 1 - kl) - row) * D) * 2u;
    }
  }
  auto copy_v = [&](int key0, uint8_t* dst) __attribute__((always_inline)) {
    const uint16_t* base = Vh + (size_t)key0 * D;
    const bool full = key0 + C::BK <= Nk;
#pragma unroll
    for (int c = 0; c < C::LOADS; ++c)
      dcopy16(base, full ? offd[c] : offr[c],
              (uint32_t)(uintptr_t)(const LDS_AS void*)(dst + c * 1024));
  };
  auto load_k = [&](int key0, bf16x8 (&kr)[C::KS]) __attribute__((always_inline)) {
    const uint16_t* kp = Kh + (size_t)min(key0 + l32, Nk - 1) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kr[ks] = __builtin_bit_cast(bf16x8, ld_global_16B(kp + ks * 16));
  };

  // Queries as B operands of S^T (k-slots = head dim).
  bf16x8 qreg[C::KS];
  {
    const uint16_t* qp = Q + ((size_t)bh * Nq + qc) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, ld_global_16B(qp + ks * 16));
  }
  // Transposing V reads: lane (group g, source s) points at row 4*hi + s/4
  // (plus 16t + 8*half) and columns 32*db + 16*(g&1) + 4*(s&3)..+3.
  int voff[C::DB];
  {
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      voff[db] = dv_off<D>(4 * hi + (sl >> 2), 32 * db + 16 * (g & 1) + 4 * (sl & 3));
  }

  f32x16 oacc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;   // running max (log2 units, scaled) of this lane's query
  float l_run = 0.f;         // running sum over this lane's half of the keys

  bf16x8 kcur[C::KS], knext[C::KS];
  if (nt > 0) {
    load_k(k_lo, kcur);
    copy_v(k_lo, v_lds[0]);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  for (int j = 0; j < nt; ++j) {
    const int key0 = k_lo + j * C::BK;
    const uint8_t* vt = v_lds[j & 1];
    // Next step's K (registers) and V (the other LDS buffer; single wave, so
    // no barrier: this wave finished reading it in the previous step).
    if (j + 1 < nt) {
      load_k(key0 + C::BK, knext);
      copy_v(key0 + C::BK, v_lds[(j + 1) & 1]);
    }
    // S^T (32 keys x 32 queries), scaled into log2 units.
    f32x16 s = zero16();
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) s = mfma_32x32x16(kcur[ks], qreg[ks], s);
    // Mask keys past this split or past the query's position.
    const bool masked = key0 + C::BK > k_hi || (CAUSAL && key0 + C::BK - 1 > Nk - Nq);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] *= c2;
      if (masked) {
        const int key = key0 + 8 * (i >> 2) + 4 * hi + (i & 3);
        s[i] = (key >= k_hi || (CAUSAL && key > qpos)) ? -INFINITY : s[i];
      }
    }
    float tmax = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) tmax = vmax(tmax, s[i]);
    tmax = halves_max(tmax);
    const float m_new = vmax(m_run, tmax);
    if (m_new > m_run) {   // per lane; a query with no admissible key keeps -inf
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = fast_exp2(s[i] - m_use);
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ls += s[i];
    l_run += ls;
    // O^T += V^T P^T over two 16-key groups (k-slot s of half h is key
    // 8*(s/4) + 4h + s%4 of the group in both operands).
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r0 = 8 * t;
      const bf16x8 pb = pack_bf16x8(s[r0], s[r0 + 1], s[r0 + 2], s[r0 + 3], s[r0 + 4], s[r0 + 5],
                                    s[r0 + 6], s[r0 + 7]);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const uint8_t* vp = vt + 16 * t * C::RB + voff[db];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)vp);
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vp + 8 * C::RB));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = mfma_32x32x16(a, pb, oacc[db]);
      }
    }
    // This step's data is consumed; wait for the next step's loads.
    __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kcur[ks] = knext[ks];
  }

  // Partial result of this split: O normalised by its own l, LSE natural.
  // A query with no admissible key here gets LSE = -inf and O = 0.
  const float l_tot = halves_sum(l_run);
  if (q < Nq) {
    const size_t row = ((size_t)bh * nsplit + sp) * Nq + q;
    const bool live = l_tot > 0.f;
    const float inv = live ? 1.f / l_tot : 0.f;
    float* orow = Opart + row * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hi;
        f32x4 v4 = {oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                    oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + d0) = v4;
      }
    if (hi == 0) Lpart[row] = live ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

// Merge of the splits for one (head, query) per workgroup of D threads.
template <int D>
__global__ __launch_bounds__(D) void fa_decode_merge_kernel(
    const float* __restrict__ Opart, const float* __restrict__ Lpart, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int Nq, int nsplit) {
  const int r = blockIdx.x;                  // bh * Nq + q
  const int bh = r / Nq, q = r % Nq;
  const int c = threadIdx.x;
  const float* lp = Lpart + (size_t)bh * nsplit * Nq + q;
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = vmax(m, lp[(size_t)s * Nq]);
  float l = 0.f, acc = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float ls = lp[(size_t)s * Nq];
    if (ls == -INFINITY) continue;
    const float wgt = fast_exp2((ls - m) * kLog2e);
    l += wgt;
    acc += wgt * Opart[(((size_t)bh * nsplit + s) * Nq + q) * D + c];
  }
  O[(size_t)r * D + c] = (uint16_t)(pack_bf16x2(acc / l, 0.f) & 0xffffu);
  if (c == 0) LSE[r] = m + fast_log2(l) * kLn2;
}

}  // namespace

// Number of key splits for a decode call: about 2048 workgroups in total
// (eight waves on each of the 256 CUs), at least 256 keys per split.
int decode_splits(int BH, int Nk, int* chunk) {
  constexpr int BK = 32;
  int ns = (2048 + BH - 1) / BH;
  const int max_ns = (Nk + 255) / 256;
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  int ch = (Nk + ns - 1) / ns;
  ch = (ch + BK - 1) / BK * BK;
  ns = (Nk + ch - 1) / ch;
  *chunk = ch;
  return ns;
}

hipError_t decode_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           float* lse, float* ws, int BH, int Nq, int Nk, int d, float scale,
                           bool causal, hipStream_t stream) {
  int chunk = 0;
  const int ns = decode_splits(BH, Nk, &chunk);
  float* opart = ws;
  float* lpart = ws + (size_t)BH * ns * Nq * d;
  const float c2 = scale * kLog2e;
  dim3 grid((unsigned)(BH * ns)), block(64);
#define FA_DEC_CASE(DD, CC)                                                                   \
  if (d == DD && causal == CC)                                                                \
    hipLaunchKernelGGL((fa_decode_kernel<DD, CC>), grid, block, 0, stream, q, k, v, opart,   \
                       lpart, Nq, Nk, ns, chunk, c2);
  FA_DEC_CASE(128, true)
  FA_DEC_CASE(128, false)
  FA_DEC_CASE(64, true)
  FA_DEC_CASE(64, false)
#undef FA_DEC_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 mgrid((unsigned)(BH * Nq));
  if (d == 128)
    hipLaunchKernelGGL((fa_decode_merge_kernel<128>), mgrid, dim3(128), 0, stream, opart, lpart,
                       o, lse, Nq, ns);
  else
    hipLaunchKernelGGL((fa_decode_merge_kernel<64>), mgrid, dim3(64), 0, stream, opart, lpart,
                       o, lse, Nq, ns);
  return hipGetLastError();
}

}  // namespace fa
