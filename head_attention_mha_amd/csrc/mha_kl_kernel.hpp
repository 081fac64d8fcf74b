// Fused attention KL divergence ("StreamKL") for gfx950: per query row
//
//   KL_i = sum_j P1_ij (log P1_ij - log P2_ij),   P_t = softmax(scale Q_t K_t^T)
//
// in one pass over the keys, without materialising either Nq x Nk matrix
// ("StreamKL", Methodology section 1). Each row keeps five running scalars:
// reference maxima m1, m2 of the two score rows, the sums l1, l2 of
// exp(S_t - m_t) and acc = sum_j exp(S1_ij - m1)(S1_ij - S2_ij), all rescaled
// when a maximum outgrows its reference by more than 2^8 (exp2 domain; the
// block maxima are taken only for blocks whose weights sum past that
// bound); at the end KL = acc / l1 + LSE2 - LSE1 with LSE_t = m_t + log l_t. There is no P.V product: acc is one number per row,
// not a row of an output matrix.
//
// Structure as the row-parallel kernels of this library: 4 waves per
// workgroup, 32 query rows per wave with both rows' Q fragments held in
// registers as MFMA B operands; tiles of 64 keys of K1 and K2 reach LDS by
// buffer loads that write LDS directly, double-buffered, one barrier per
// tile. S_t^T = K_t Q_t^T puts the query on the MFMA columns, so each lane
// owns one query row (two lanes per row, one per half of the keys, merged
// with a cross-half exchange). Causal tiles past the frontier are skipped
// (the page's causal handling); only diagonal and tail tiles carry an element
// mask. The maxima are kept on the raw scores and the sums in the exp2
// domain (scores times scale * log2(e)), the scale entering each exponent
// through one fused multiply-add.
#pragma once

#include "mha_fwd_kernel.hpp"
#include "mha_sync.hpp"

namespace mha {

struct KlParams {
  const uint16_t* q1;
  const uint16_t* k1;
  const uint16_t* q2;
  const uint16_t* k2;
  float* kl;
  float* lse1;
  float* lse2;
  int B, H, Nq, Nk;
  float scale;       // softmax scale of both distributions (> 0)
  float scale_log2;  // scale * log2(e)
  float defer_raw;   // rescale threshold in raw-score units: 8 / scale_log2
  int n_blocks;      // workgroups launched
  int n_tiles;       // query blocks per (b, h)
};

namespace kl {
// kWaves, kThreads, kBQ (query rows per workgroup) and kBK (keys per tile)
// are in mha_tiles.hpp
constexpr float kLn2 = 0.69314718055994531f;
// Maximum over the two halves of the wave (lanes l and l ^ 32), as a
// three-input maximum from -inf
__device__ __forceinline__ float max_halves3(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  const uint32_t lo = r[0], hi = r[1];
  return fmaxf(fmaxf(-__builtin_inff(), __builtin_bit_cast(float, lo)), __builtin_bit_cast(float, hi));
}
}  // namespace kl

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kl::kThreads) void mha_kl_kernel(KlParams p) {
  using O_ = Ops<T>;
  constexpr int BK = kl::kBK;
  constexpr int kBQ = kl::kBQ;
  constexpr int NW = kl::kWaves;
  constexpr int KB = BK / 32;            // 32-key blocks per tile
  constexpr int DK = D / 16;             // k-steps over the head dim
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BK * ROWB;
  constexpr int RPI = 1024 / ROWB;
  constexpr int NCPW = TILEB / 1024 / NW;  // 1 KiB copies per wave per tensor
  static_assert(NCPW >= 1 && (NW * RPI) % 16 == 0, "copy layout");
  constexpr float NEG_INF = -__builtin_inff();

  __shared__ __attribute__((aligned(1024))) uint8_t lds_a0[TILEB];  // K1, buffer 0
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a1[TILEB];  // K1, buffer 1
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b0[TILEB];  // K2, buffer 0
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b1[TILEB];  // K2, buffer 1

  // work item: (batch, head, query block); a head's blocks on one XCD when
  // the heads split evenly over the 8 XCDs, heaviest causal blocks first
  const int lin = blockIdx.x;
  const int BH = p.B * p.H;
  const bool by_xcd = (BH & 7) == 0;
  const int nh = by_xcd ? BH >> 3 : BH;
  // two workgroups per CU
  const int kk = by_xcd ? engine_order(lin >> 3, nh * p.n_tiles, 64) : lin;
  const int qi = kk / nh;
  const int hh = kk - qi * nh;
  const int bh = by_xcd ? 8 * hh + (lin & 7) : hh;
  const int qt = CAUSAL ? p.n_tiles - 1 - qi : qi;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int q0 = qt * kBQ;

  const size_t rs = (size_t)p.H * D;
  const size_t qo = ((size_t)b * p.Nq * p.H + h) * D;
  const size_t kvo = ((size_t)b * p.Nk * p.H + h) * D;
  const uint32_t row_bytes = (uint32_t)(rs * 2);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + ln;

  // Q1 and Q2 fragments of this lane's query row (B operands), read once
  u32x4 q1f[DK], q2f[DK];
  if (my_q < p.Nq) {
    const uint16_t* r1 = p.q1 + qo + (size_t)my_q * rs + 8 * hf;
    const uint16_t* r2 = p.q2 + qo + (size_t)my_q * rs + 8 * hf;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      q1f[i] = *reinterpret_cast<const u32x4*>(r1 + 16 * i);
      q2f[i] = *reinterpret_cast<const u32x4*>(r2 + 16 * i);
    }
  } else {
#pragma unroll
    for (int i = 0; i < DK; ++i) q1f[i] = q2f[i] = u32x4{0, 0, 0, 0};
  }

  // key tiles: [0, jm) need no mask, [jm, j_end) need one, [j_end, n_kt)
  // are past this wave's rows
  const int n_ktiles_all = (p.Nk + BK - 1) / BK;
  int n_kt = n_ktiles_all;
  if (CAUSAL) n_kt = min(n_ktiles_all, (min(p.Nq, q0 + kBQ) + BK - 1) / BK);
  int jm = (p.Nk % BK) ? p.Nk / BK : n_ktiles_all;
  if (CAUSAL) jm = min(jm, (qw0 + 1) / BK);
  int j_end = CAUSAL ? min(n_kt, qw0 / BK + 1) : n_kt;
  if (qw0 >= p.Nq) j_end = 0;
  jm = min(jm, j_end);

  uint32_t c_off[NCPW];
#pragma unroll
  for (int c = 0; c < NCPW; ++c) {
    const int row = (c * NW + wave) * RPI + lane / CH;
    c_off[c] = row * row_bytes + 16 * ((lane % CH) ^ k_swz<D>(row));
  }
  auto issue = [&](int j, uint8_t* la, uint8_t* lb) __attribute__((always_inline)) {
    const int nvalid = min(BK, p.Nk - j * BK);
    const uint32_t bytes = (uint32_t)(nvalid - 1) * row_bytes + ROWB;
    const auto r1 = make_rsrc(p.k1 + kvo + (size_t)j * BK * rs, bytes);
    const auto r2 = make_rsrc(p.k2 + kvo + (size_t)j * BK * rs, bytes);
#pragma unroll
    for (int c = 0; c < NCPW; ++c) dma16(r1, la + (c * NW + wave) * 1024, c_off[c]);
#pragma unroll
    for (int c = 0; c < NCPW; ++c) dma16(r2, lb + (c * NW + wave) * 1024, c_off[c]);
  };

  uint32_t roff[DK];
  {
    const int key = k_row_order(ln);
    const int sw = k_swz<D>(key);
#pragma unroll
    for (int i = 0; i < DK; ++i) roff[i] = key * ROWB + 16 * ((2 * i + hf) ^ sw);
  }

  // running state of this lane's half of the row (m shared by both halves):
  // reference maxima of the raw scores, sums in the exp2 domain relative to
  // m * c, acc = sum exp2((S1 - m1) c) (S1 - S2) over raw score
  // differences. As in the forward, the rescale is deferred: the reference
  // maxima move only when a block's maximum exceeds them by more than 2^8
  // in the exp2 domain, so the weights stay below 2^8 and most blocks skip
  // the rescale. Each sum runs in two chains (even and odd elements).
  float m1 = NEG_INF, m2 = NEG_INF;
  float m1c = 0.f, m2c = 0.f;  // m * c, 0 while m = -inf (no key seen yet)
  float l1[2] = {0.f, 0.f}, l2[2] = {0.f, 0.f}, acc[2] = {0.f, 0.f};
  const float c = p.scale_log2;

  // One 32-key block at a time, so that only one block's S1^T and S2^T
  // accumulators are live.
  auto tile_body = [&](int j, const uint8_t* la, const uint8_t* lb, auto mask_tag)
                       __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      // S1^T = K1 Q1^T and S2^T = K2 Q2^T, keys on the MFMA rows
      f32x16 s1, s2;
#pragma unroll
      for (int r = 0; r < 16; ++r) s1[r] = s2[r] = 0.f;
#pragma unroll
      for (int i = 0; i < DK; ++i) {
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(la + roff[i] + kb * 32 * ROWB);
        const u32x4 a2 = *reinterpret_cast<const u32x4*>(lb + roff[i] + kb * 32 * ROWB);
        s1 = O_::mfma(a1, q1f[i], s1);
        s2 = O_::mfma(a2, q2f[i], s2);
      }
      sync::PinReads<0, 2 * DK, 1, 4>::apply();
      __builtin_amdgcn_sched_barrier(0);
      // raw scores; element r is key j*BK + 32*kb + 16*(r>>3) + 8*hf + (r&7).
      // The maxima are taken on the raw scores (the scale is positive) and
      // the scale enters once, inside each exponent's fused multiply-add.
      float x1[16], x2[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x1[r] = s1[r];
        x2[r] = s2[r];
      }
      if constexpr (MASK) {
        // visible iff key < Nk and (causal) key <= my_q: one per-lane limit
        // on the element's offset 16*(r>>3) + (r&7), a constant
        const int lim = (CAUSAL ? min(p.Nk - 1, my_q) : p.Nk - 1) - j * BK - kb * 32 - 8 * hf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool vis = 16 * (r >> 3) + (r & 7) <= lim;
          x1[r] = vis ? x1[r] : NEG_INF;
          x2[r] = vis ? x2[r] : NEG_INF;
        }
      }
      // The exact step: block maxima (chains started from -inf, so that the
      // compiler forms three-input maxima throughout, with no NaN-quieting
      // copies of the raw scores), merged over the two halves, and the
      // deferred rescale of whichever distribution's maximum outgrew its
      // reference by more than the bound.
      auto max_and_rescale = [&]() __attribute__((always_inline)) {
        float t1 = NEG_INF, t2 = NEG_INF;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          t1 = fmaxf(t1, x1[r]);
          t2 = fmaxf(t2, x2[r]);
        }
        t1 = kl::max_halves3(t1);
        t2 = kl::max_halves3(t2);
        // A row that sees no key of this block (causal, diagonal tile) has
        // t = -inf and never moves its maximum here; while a row has seen no
        // key at all its m * c stays 0, so masked weights are exp2(-inf) = 0.
        const bool g1 = t1 > m1 + p.defer_raw, g2 = t2 > m2 + p.defer_raw;
        if (__any(g1 || g2)) {
          // the wave-uniform branch is rare after the first blocks
          asm volatile("" ::: "memory");
          if (g1) {
            const float al = fast_exp2((m1 - t1) * c);  // 0 when m1 = -inf
            m1 = t1;
            m1c = t1 * c;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              l1[e] *= al;
              acc[e] *= al;
            }
          }
          if (g2) {
            const float al = fast_exp2((m2 - t2) * c);
            m2 = t2;
            m2c = t2 * c;
#pragma unroll
            for (int e = 0; e < 2; ++e) l2[e] *= al;
          }
        }
      };
      // The block's weights against the reference maxima, summed in two
      // chains each (even and odd elements) that start from the block's
      // first elements; the raw scores stay as they are.
      float b1[2], b2[2], ba[2];
      auto block_sums = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p1 = fast_exp2(__builtin_fmaf(x1[r], c, -m1c));
          const float p2 = fast_exp2(__builtin_fmaf(x2[r], c, -m2c));
          // the difference of the raw (unmasked, finite) scores; the scale
          // is applied to acc once at the end. Exactly 0 where the two
          // scores are equal.
          const float dx = s1[r] - s2[r];
          if (r < 2) {
            b1[r] = p1;
            b2[r] = p2;
            ba[r] = p1 * dx;
          } else {
            b1[r & 1] += p1;
            b2[r & 1] += p2;
            ba[r & 1] = __builtin_fmaf(p1, dx, ba[r & 1]);
          }
        }
      };
      // The maxima only decide whether a reference moves, i.e. whether some
      // score exceeds it by more than the deferral bound. Every weight is at
      // most its lane's block sum, so sums within 2^kDeferLog2 on every lane
      // show that no score crossed the bound and the maxima are not needed.
      // Otherwise the exact step runs and the block is summed again; so
      // does the first block, which sets both references (every row sees
      // key 0). The test is written so that a NaN or infinite sum fails it.
      bool exact = kb == 0 && j == 0;
      if (!exact) {
        block_sums();
        exact = __any(!(b1[0] + b1[1] <= kDeferSum) || !(b2[0] + b2[1] <= kDeferSum));
      }
      if (exact) {
        max_and_rescale();
        block_sums();
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        l1[e] += b1[e];
        l2[e] += b2[e];
        acc[e] += ba[e];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto step = [&](int j, auto par, auto mode) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    constexpr int MODE = decltype(mode)::value;  // 0 idle, 1 masked, 2 unmasked
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    sync::bare_barrier();
    if (j + 1 < n_kt) {
      if constexpr (P == 0) issue(j + 1, lds_a1, lds_b1);
      else issue(j + 1, lds_a0, lds_b0);
    }
    if constexpr (MODE != 0) {
      using M = std::integral_constant<bool, MODE == 1>;
      if constexpr (P == 0) tile_body(j, lds_a0, lds_b0, M{});
      else tile_body(j, lds_a1, lds_b1, M{});
    }
  };
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  auto run = [&](int j0, int j1, auto mode) __attribute__((always_inline)) {
    int j = j0;
    if (j < j1 && (j & 1)) step(j++, Odd{}, mode);
    for (; j + 1 < j1; j += 2) {
      step(j, Even{}, mode);
      step(j + 1, Odd{}, mode);
    }
    if (j < j1) step(j, Even{}, mode);
  };
  if (n_kt > 0) issue(0, lds_a0, lds_b0);
  run(0, jm, std::integral_constant<int, 2>{});
  run(jm, j_end, std::integral_constant<int, 1>{});
  run(j_end, n_kt, std::integral_constant<int, 0>{});

  // both halves of the row: add the sums, then KL = acc/l1 + LSE2 - LSE1
  const float L1 = sum_halves(l1[0] + l1[1]);
  const float L2 = sum_halves(l2[0] + l2[1]);
  const float A = sum_halves(acc[0] + acc[1]);
  if (hf == 0 && my_q < p.Nq) {
    const float lse1 = __builtin_fmaf(m1, c, fast_log2(L1)) * kl::kLn2;
    const float lse2 = __builtin_fmaf(m2, c, fast_log2(L2)) * kl::kLn2;
    const size_t r = (size_t)bh * p.Nq + my_q;
    p.lse1[r] = lse1;
    p.lse2[r] = lse2;
    // LSE2 - LSE1 from the differences of the maxima and of the log sums,
    // not of the two LSEs (no cancellation of two large values, and exactly
    // 0 for identical distributions)
    const float dlse = (m2 - m1) * c + (fast_log2(L2) - fast_log2(L1));
    p.kl[r] = (A * c / L1 + dlse) * kl::kLn2;
  }
}

}  // namespace mha
