// Output projection after attention on gfx950: Y = concat_heads(O) W^T (+ b).
//
// The attention output O [B, Nq, H, d] already is the head concatenation
// ("SparkAttention", MHA-Forward passage, Eq. 1: heads concatenated, then
// multiplied by W_O) once read as X [M = B*Nq, K = H*d]; the projection is
// the matrix product Y [M, N] = X W^T with W [N, K] (one output feature per
// row) and an optional bias. No reshuffle of O is needed.
//
// MFMA kernel (32x32x16, fp32 accumulation). The product is formed
// transposed, Y^T = W X^T: W rows are the A operand and X rows the B
// operand, both 16-byte row reads from LDS, and the accumulator holds four
// consecutive output features per lane and register group, so Y is stored
// in 8-byte pieces. Workgroup: 8 waves, a 256 (features) x 256 (tokens)
// tile; each wave 128 x 64 (4 x 2 MFMA blocks). K advances 64 at a time
// through double-buffered LDS stages filled by buffer loads that write LDS
// directly (one barrier per stage). Rows past M or N read as zero and are
// not stored.
#pragma once

#include "mha_fwd_kernel.hpp"
#include "mha_sync.hpp"

namespace mha {

struct ProjParams {
  const uint16_t* x;   // [M, K]
  const uint16_t* w;   // [N, K]
  const uint16_t* bias;  // [N] or null
  uint16_t* y;         // [M, N]
  int M, N, K;
  int tiles_n;         // ceil(N / 256)
  int n_tiles;         // tiles_n * ceil(M / 256)
};

namespace proj {
// kWaves, kThreads, kBN (output features per workgroup), kBM (tokens per
// workgroup) and kBK (K per stage) are in mha_tiles.hpp

// 16-byte-chunk swizzle of the 128-byte stage rows: 8 consecutive rows, and
// the 8 rows of each parity among 16 consecutive rows, use 8 different
// chunk positions, so the MFMA row reads are conflict-free for 128- and
// 256-byte LDS passes.
__device__ __forceinline__ int g_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
}  // namespace proj

template <typename T>
__global__ __launch_bounds__(proj::kThreads) void mha_proj_kernel(ProjParams p) {
  using O_ = Ops<T>;
  constexpr int NW = proj::kWaves;
  constexpr int ROWB = proj::kBK * 2;          // 128 bytes per stage row
  constexpr int STAGEB = proj::kBN * ROWB;     // 32 KiB per operand per stage
  constexpr int NCPW = STAGEB / 1024 / NW;     // 1 KiB copies per wave per operand (4)
  constexpr int RPC = 1024 / ROWB;             // rows per 1 KiB copy (8)
  constexpr int EB = 4, TB = 2;                // MFMA blocks per wave (features, tokens)

  __shared__ __attribute__((aligned(1024))) uint8_t lw0[STAGEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lw1[STAGEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lx0[STAGEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lx1[STAGEB];

  // tile: consecutive tiles share a token block; with whole groups of 8,
  // each XCD takes a contiguous run of tiles
  const int lin = blockIdx.x;
  const int tile = (p.n_tiles & 7) == 0 ? (lin & 7) * (p.n_tiles >> 3) + (lin >> 3) : lin;
  const int tm = tile / p.tiles_n;
  const int tn = tile - tm * p.tiles_n;
  const int n0 = tn * proj::kBN, m0 = tm * proj::kBM;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int we = wave & 1;   // feature half of the tile
  const int wt = wave >> 1;  // token quarter of the tile
  const uint32_t row_bytes = (uint32_t)p.K * 2;

  // stage copies: copy c of this wave covers rows (c*NW + wave)*RPC + lane/8
  uint32_t c_off[NCPW];
#pragma unroll
  for (int c = 0; c < NCPW; ++c) {
    const int row = (c * NW + wave) * RPC + lane / 8;
    c_off[c] = row * row_bytes + 16 * ((lane % 8) ^ proj::g_swz(row));
  }
  const int nvw = min(proj::kBN, p.N - n0), nvx = min(proj::kBM, p.M - m0);
  const uint32_t bytes_w = (uint32_t)(nvw - 1) * row_bytes + ROWB;
  const uint32_t bytes_x = (uint32_t)(nvx - 1) * row_bytes + ROWB;
  auto issue = [&](int s, uint8_t* lw, uint8_t* lx) __attribute__((always_inline)) {
    const int k0 = s * proj::kBK;
    const auto rw = make_rsrc(p.w + (size_t)n0 * p.K + k0, bytes_w);
    const auto rx = make_rsrc(p.x + (size_t)m0 * p.K + k0, bytes_x);
#pragma unroll
    for (int c = 0; c < NCPW; ++c) dma16(rw, lw + (c * NW + wave) * 1024, c_off[c]);
#pragma unroll
    for (int c = 0; c < NCPW; ++c) dma16(rx, lx + (c * NW + wave) * 1024, c_off[c]);
  };

  // read offsets: lane reads row ln of each 32-row block at chunk 2*ks + hf
  uint32_t woff[EB][4], xoff[TB][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      const int row = we * 128 + eb * 32 + ln;
      woff[eb][ks] = row * ROWB + 16 * ((2 * ks + hf) ^ proj::g_swz(row));
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int row = wt * 64 + tb * 32 + ln;
      xoff[tb][ks] = row * ROWB + 16 * ((2 * ks + hf) ^ proj::g_swz(row));
    }
  }

  f32x16 acc[EB][TB];
#pragma unroll
  for (int eb = 0; eb < EB; ++eb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[eb][tb][r] = 0.f;

  // All MFMAs of a stage in k-step order; the six operands of k-step ks + 1
  // are read while the eight MFMAs of k-step ks issue (pinned below), so
  // LDS latency hides behind MFMA work after the first k-step.
  auto compute = [&](const uint8_t* lw, const uint8_t* lx) __attribute__((always_inline)) {
    constexpr int NKS = 4;
    u32x4 wa[2][EB], xb[2][TB];
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) wa[0][eb] = *reinterpret_cast<const u32x4*>(lw + woff[eb][0]);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) xb[0][tb] = *reinterpret_cast<const u32x4*>(lx + xoff[tb][0]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int c = ks & 1;
      if (ks + 1 < NKS) {
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) wa[c ^ 1][eb] = *reinterpret_cast<const u32x4*>(lw + woff[eb][ks + 1]);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) xb[c ^ 1][tb] = *reinterpret_cast<const u32x4*>(lx + xoff[tb][ks + 1]);
      }
#pragma unroll
      for (int eb = 0; eb < EB; ++eb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[eb][tb] = O_::mfma(wa[c][eb], xb[c][tb], acc[eb][tb]);
    }
    // pins: the first k-step's reads, then per k-step its MFMAs with the
    // next k-step's reads spread among them (one read after each MFMA but
    // the last two)
    __builtin_amdgcn_sched_group_barrier(0x100, EB + TB, 0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int m = 0; m < EB * TB; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (ks + 1 < NKS && m < EB + TB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };
  const int n_stages = p.K / proj::kBK;
  auto step = [&](int s, auto par) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    sync::bare_barrier();
    if (s + 1 < n_stages) {
      if constexpr (P == 0) issue(s + 1, lw1, lx1);
      else issue(s + 1, lw0, lx0);
    }
    if constexpr (P == 0) compute(lw0, lx0);
    else compute(lw1, lx1);
  };
  issue(0, lw0, lx0);
  int s = 0;
  for (; s + 1 < n_stages; s += 2) {
    step(s, std::integral_constant<int, 0>{});
    step(s + 1, std::integral_constant<int, 1>{});
  }
  if (s < n_stages) step(s, std::integral_constant<int, 0>{});

  // epilogue: lane = token, register group a = 4 consecutive features
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int t = m0 + wt * 64 + tb * 32 + ln;
    if (t >= p.M) continue;
    uint16_t* yrow = p.y + (size_t)t * p.N;
#pragma unroll
    for (int eb = 0; eb < EB; ++eb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int e = n0 + we * 128 + eb * 32 + 8 * a + 4 * hf;
        if (e >= p.N) continue;
        float v0 = acc[eb][tb][4 * a], v1 = acc[eb][tb][4 * a + 1];
        float v2 = acc[eb][tb][4 * a + 2], v3 = acc[eb][tb][4 * a + 3];
        if (p.bias) {
          const u32x2 bb = *reinterpret_cast<const u32x2*>(p.bias + e);
          const uint32_t b01 = bb[0], b23 = bb[1];
          f32x2 f01, f23;
          if constexpr (std::is_same<T, BF16>::value) {
            f01 = f32x2{__builtin_bit_cast(float, b01 << 16), __builtin_bit_cast(float, b01 & 0xffff0000u)};
            f23 = f32x2{__builtin_bit_cast(float, b23 << 16), __builtin_bit_cast(float, b23 & 0xffff0000u)};
          } else {
            f01 = __builtin_convertvector(__builtin_bit_cast(f16x2, b01), f32x2);
            f23 = __builtin_convertvector(__builtin_bit_cast(f16x2, b23), f32x2);
          }
          v0 += f01[0];
          v1 += f01[1];
          v2 += f23[0];
          v3 += f23[1];
        }
        u32x2 w2;
        w2[0] = O_::pack(v0, v1);
        w2[1] = O_::pack(v2, v3);
        *reinterpret_cast<u32x2*>(yrow + e) = w2;
      }
  }
}

}  // namespace mha
