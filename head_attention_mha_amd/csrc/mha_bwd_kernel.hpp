// Attention backward for gfx950 (CDNA4): dQ, dK and dV of the fused forward.
//
// The forward is recomputed tile by tile from the stored LSE, P = exp(S -
// LSE) ("StreamKL", Methodology section 2), never materialising the Nq x Nk
// matrices. With D_i = sum_c dO_ic O_ic (the per-row term the SparkAttention
// backward passage calls dPsum) the gradients are
//
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Three kernels, each owning its outputs (no atomics, no workspace):
// * mha_bwd_dkdv_kernel: column-parallel, as the pages' backward workers are
//   (the FlashAttention long-sequence post, "Attention parallelism"; the
//   SparkAttention backward passage): each wave owns 32 keys, streams the
//   Q/dO tiles that see them and accumulates their dK and dV in registers.
//   At d = 128, mha_bwd_dkdv_pair_kernel does the same work with two waves
//   per 32 keys (a producer of P and dS and a consumer accumulating dK and
//   dV), so that two waves share each SIMD.
// * mha_bwd_dq_kernel: row-parallel, like the forward: each wave owns 32
//   query rows and streams K/V tiles. The pages add dQ across column workers
//   with atomics; "StreamKL" (Methodology section 2) also describes separate
//   kernels for when the dQ buffer does not fit in L2. Separate kernels are
//   used here always: S and dP are computed once more, but dQ needs neither
//   atomics nor an fp32 buffer, and the result is deterministic.
//
// Layouts mirror the forward so that no operand needs a cross-lane move:
// the score tile is computed with the query (dq) or key (dkdv) index on the
// MFMA columns, i.e. one query/key per lane, and the rows of the other
// operand are fed in the order of k_row_order, which leaves every lane
// holding 8 consecutive keys/queries per 16-step -- exactly the B-operand
// fragment of the following product. The transposed operands (K^T for dQ,
// dO^T and Q^T for dV and dK) come from gfx950 LDS transpose reads.
#pragma once

#include "mha_fwd_kernel.hpp"
#include "mha_sync.hpp"

namespace mha {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;
  int B, H, Nq, Nk;
  float scale;       // softmax scale (> 0)
  float scale_log2;  // scale * log2(e)
  int n_blocks;      // workgroups launched
  int n_tiles;       // query blocks (dq) or key blocks (dkdv) per (b, h)
};

namespace bwd {

// kWaves, kThreads, kBQ (query rows per dq workgroup), kBKV (keys per dkdv
// workgroup), kBK (keys per dq tile) and kBQt (queries per dkdv tile) are in
// mha_tiles.hpp
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDkdvAhead = 4;  // dK/dV operand reads issued this many MFMAs ahead

using mha::lds_read_tr16;
using mha::t_swz;
using mha::tr_off;
using mha::tr_operand;

// Two packed 16-bit values -> fp32.
template <typename T>
__device__ __forceinline__ f32x2 unpack2(uint32_t w) {
  if constexpr (std::is_same<T, BF16>::value) {
    return f32x2{__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u)};
  } else {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
  }
}

// One wave copies 256 bytes global -> LDS: lane l's 4 bytes at `voffset`
// land at lds_dst + 4*l (per-dword range check: lanes past the end get 0).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds_dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)((lds_u8*)lds_dst),
                                           4, voffset, 0, 0, 0);
}

// Calls f(std::integral_constant<int, I>) for I = B, ..., E - 1 in order.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Element ranges of VALU work spread over fenced slots: slot j of a tile
// handles elements [lo(j), lo(j + 1)) of a 16-element task spread evenly
// over slots [FIRST, FIRST + COUNT). A packed pair may straddle two slots.
template <int FIRST, int COUNT>
struct Spread {
  static constexpr __host__ __device__ int lo(int j) {
    return j <= FIRST ? 0 : j >= FIRST + COUNT ? 16 : (16 * (j - FIRST)) / COUNT;
  }
};

// Query-side mask of a dK/dV tile. The lane's element r is query
// qt0 + 8*hf + o with o = 16*(r>>3) + (r&7), a constant; it is visible iff
// the query exists and (causal) does not precede the lane's key, i.e. iff o
// lies in [lo, hi]. Held as a start and a width, so that one unsigned compare
// of o - start decides it; an empty range gets a start no offset reaches.
template <bool CAUSAL>
struct QueryMask {
  int start;
  uint32_t width;
  __device__ __forceinline__ QueryMask(int qt0, int hf, int my_k, int Nq) {
    const int hi = Nq - 1 - qt0 - 8 * hf;
    const int lo = CAUSAL ? my_k - qt0 - 8 * hf : 0;
    start = hi >= lo ? lo : (1 << 30);
    width = hi >= lo ? (uint32_t)(hi - lo) : 0u;
  }
  __device__ __forceinline__ bool visible(int o) const { return (uint32_t)(o - start) <= width; }
};

}  // namespace bwd

// ---- dQ: row-parallel ----------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(bwd::kThreads) void mha_bwd_dq_kernel(BwdParams p) {
  using O_ = Ops<T>;
  constexpr int BK = bwd::kBK;
  constexpr int kBQ = bwd::kBQ;
  constexpr int NW = bwd::kWaves;
  constexpr int KB = BK / 32;            // 32-key blocks per tile
  constexpr int DK = D / 16;             // k-steps over the head dim
  constexpr int DB = D / 32;             // 32-row blocks of dQ^T
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BK * ROWB;
  constexpr int RPI = 1024 / ROWB;
  constexpr int NCPW = TILEB / 1024 / NW;  // 1 KiB copies per wave per tensor
  static_assert(NCPW >= 1 && (NW * RPI) % 16 == 0, "copy layout");

  __shared__ __attribute__((aligned(1024))) uint8_t lds_k0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v1[TILEB];

  // work item: (batch, head, query block); a head's blocks on one XCD when
  // the heads split evenly over the 8 XCDs, heaviest causal blocks first
  const int lin = blockIdx.x;
  const int BH = p.B * p.H;
  const bool by_xcd = (BH & 7) == 0;
  const int nh = by_xcd ? BH >> 3 : BH;
  // two (d = 128) or three (d = 64) workgroups per CU
  const int kk = by_xcd ? engine_order(lin >> 3, nh * p.n_tiles, D == 128 ? 64 : 96) : lin;
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

  // Q and dO fragments (B operands), read once; LSE (log2 units); and
  // D = rowsum(dO o O), formed here from the same elements of O as the lane
  // holds of dO (half a row: lanes l and l ^ 32 share a row) and written
  // out for the dK/dV kernel, which runs after this one
  u32x4 qf[DK], gf[DK];
  float lse2 = 0.f, dpart = 0.f;
  if (my_q < p.Nq) {
    const uint16_t* qrow = p.q + qo + (size_t)my_q * rs + 8 * hf;
    const uint16_t* grow = p.dout + qo + (size_t)my_q * rs + 8 * hf;
    const uint16_t* orow = p.o + qo + (size_t)my_q * rs + 8 * hf;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      qf[i] = *reinterpret_cast<const u32x4*>(qrow + 16 * i);
      gf[i] = *reinterpret_cast<const u32x4*>(grow + 16 * i);
      const u32x4 ov = *reinterpret_cast<const u32x4*>(orow + 16 * i);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t gw = gf[i][w], ow = ov[w];
        const f32x2 a = bwd::unpack2<T>(ow);
        const f32x2 g = bwd::unpack2<T>(gw);
        dpart = __builtin_fmaf(a[0], g[0], dpart);
        dpart = __builtin_fmaf(a[1], g[1], dpart);
      }
    }
    lse2 = p.lse[(size_t)bh * p.Nq + my_q] * bwd::kLog2e;
  } else {
#pragma unroll
    for (int i = 0; i < DK; ++i) qf[i] = gf[i] = u32x4{0, 0, 0, 0};
  }
  const float dlt = sum_halves(dpart);
  if (hf == 0 && my_q < p.Nq) p.delta[(size_t)bh * p.Nq + my_q] = dlt;

  // key tiles
  const int n_ktiles_all = (p.Nk + BK - 1) / BK;
  int n_kt = n_ktiles_all;
  if (CAUSAL) n_kt = min(n_ktiles_all, (min(p.Nq, q0 + kBQ) + BK - 1) / BK);
  int jm = (p.Nk % BK) ? p.Nk / BK : n_ktiles_all;  // tiles [0, jm) need no mask
  if (CAUSAL) jm = min(jm, (qw0 + 1) / BK);
  int j_end = CAUSAL ? min(n_kt, qw0 / BK + 1) : n_kt;  // this wave's last tile + 1
  if (qw0 >= p.Nq) j_end = 0;                               // no real rows in this wave
  jm = min(jm, j_end);

  // K and V tiles: LDS copies, rows swizzled in 16-byte chunks by t_swz
  uint32_t c_off[NCPW];
#pragma unroll
  for (int c = 0; c < NCPW; ++c) {
    const int row = (c * NW + wave) * RPI + lane / CH;
    c_off[c] = row * row_bytes + 16 * ((lane % CH) ^ bwd::t_swz<D>(row));
  }
  auto issue = [&](int j, uint8_t* lk, uint8_t* lv) __attribute__((always_inline)) {
    const int nvalid = min(BK, p.Nk - j * BK);
    const uint32_t bytes = (uint32_t)(nvalid - 1) * row_bytes + ROWB;
    const auto rk = make_rsrc(p.k + kvo + (size_t)j * BK * rs, bytes);
    const auto rv = make_rsrc(p.v + kvo + (size_t)j * BK * rs, bytes);
#pragma unroll
    for (int c = 0; c < NCPW; ++c) dma16(rk, lk + (c * NW + wave) * 1024, c_off[c]);
#pragma unroll
    for (int c = 0; c < NCPW; ++c) dma16(rv, lv + (c * NW + wave) * 1024, c_off[c]);
  };

  // LDS read offsets: row operands (K and V rows in MFMA row order) and the
  // transposed K^T operand
  uint32_t roff[DK];
  {
    const int key = k_row_order(ln);
    const int sw = bwd::t_swz<D>(key);
#pragma unroll
    for (int i = 0; i < DK; ++i) roff[i] = key * ROWB + 16 * ((2 * i + hf) ^ sw);
  }
  uint32_t toff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 2; ++r) toff[db][r] = bwd::tr_off<D>(lane, db, r);

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;
  const float c = p.scale_log2;

  // MASK: element masks (diagonal and tail tiles); a compile-time flag, so
  // that each variant of the tile body is one straight-line block
  // One 32-key block of a tile at a time, so that only one block's S^T and
  // dP^T accumulators are live.
  auto tile_body = [&](int j, const uint8_t* lk, const uint8_t* lv, auto mask_tag)
                       __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T (keys on MFMA rows, one query per lane)
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int i = 0; i < DK; ++i) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(lk + roff[i] + kb * 32 * ROWB);
        const u32x4 va = *reinterpret_cast<const u32x4*>(lv + roff[i] + kb * 32 * ROWB);
        s = O_::mfma(ka, qf[i], s);
        dp = O_::mfma(va, gf[i], dp);
      }
      sync::PinReads<0, 2 * DK, 1, 4>::apply();
      __builtin_amdgcn_sched_barrier(0);
      // P = exp(scale*s - LSE), dS = P o (dP - D); element r is key
      // j*BK + 32*kb + 16*(r>>3) + 8*hf + (r&7)
      // visible iff key < Nk and (causal) key <= my_q: one per-lane limit
      // on the element's offset 16*(r>>3) + (r&7), a constant
      const int lim = (CAUSAL ? min(p.Nk - 1, my_q) : p.Nk - 1) - j * BK - kb * 32 - 8 * hf;
      u32x4 pf[2];
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
        if constexpr (MASK) pv = 16 * (r >> 3) + (r & 7) <= lim ? pv : 0.f;
        e[r] = pv * (dp[r] - dlt);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int t = 0; t < 4; ++t) pf[half][t] = O_::pack(e[8 * half + 2 * t], e[8 * half + 2 * t + 1]);
      __builtin_amdgcn_sched_barrier(0);
      // dQ^T += K^T dS^T over this block's 32 keys
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 a = bwd::tr_operand(lk + (kb * 32 + ks * 16) * ROWB, toff[db][0], toff[db][1]);
          dq[db] = O_::mfma(a, pf[ks], dq[db]);
        }
      sync::PinReads<0, 2 * DB, 2, 4>::apply();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One barrier per tile: tile j waits for its own copies (vmcnt) and for
  // this wave's LDS reads of tile j-1 (lgkmcnt); after the barrier every
  // wave is done with tile j-1's buffers, which then take tile j+1. Tile j
  // lives in buffer j & 1. Tiles [0, jm) need no mask, [jm, j_end) need one,
  // [j_end, n_kt) are past this wave's rows. Each kind of step is a
  // straight-line body with the buffer parity fixed at compile time, so the
  // accumulators stay in place across the loop.
  auto step = [&](int j, auto par, auto mode) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    constexpr int MODE = decltype(mode)::value;  // 0 idle, 1 masked, 2 unmasked
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    sync::bare_barrier();
    if (j + 1 < n_kt) {
      if constexpr (P == 0) issue(j + 1, lds_k1, lds_v1);
      else issue(j + 1, lds_k0, lds_v0);
    }
    if constexpr (MODE != 0) {
      using M = std::integral_constant<bool, MODE == 1>;
      if constexpr (P == 0) tile_body(j, lds_k0, lds_v0, M{});
      else tile_body(j, lds_k1, lds_v1, M{});
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
  issue(0, lds_k0, lds_v0);
  run(0, jm, std::integral_constant<int, 2>{});
  run(jm, j_end, std::integral_constant<int, 1>{});
  run(j_end, n_kt, std::integral_constant<int, 0>{});

  // dQ = scale * dQ^T, rounded to the I/O type, stored as whole rows through
  // the K tile buffers (free once every wave has left the tile loop; no copy
  // is in flight)
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
  sync::bare_barrier();
  {
    const int nrows = min(kBQ, p.Nq - q0);
    const auto out = make_rsrc(p.dq + qo + (size_t)q0 * rs, (uint32_t)(nrows - 1) * row_bytes + 2 * D);
    uint8_t* const slot = (wave < 2 ? lds_k0 : lds_k1) + (wave & 1) * 32 * 2 * D;
    store_rows<O_, D>(dq, p.scale, slot, out, (uint32_t)(wave * 32) * row_bytes, row_bytes, lane);
  }
}

// ---- dK, dV: column-parallel ---------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(bwd::kThreads) void mha_bwd_dkdv_kernel(BwdParams p) {
  using O_ = Ops<T>;
  constexpr int BQt = bwd::kBQt;
  constexpr int kBKV = bwd::kBKV;
  constexpr int NW = bwd::kWaves;
  constexpr int DK = D / 16;
  constexpr int DB = D / 32;
  constexpr int PK = BQt / 16;           // 16-query steps of dV^T / dK^T
  constexpr int CH = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BQt * ROWB;      // Q or dO tile
  constexpr int RPI = 1024 / ROWB;
  constexpr int NCPW = TILEB / 1024 / NW;
  static_assert(NCPW >= 1 && (NW * RPI) % 16 == 0, "copy layout");

  // Q and dO tiles, three buffers of each. Separate objects: the compiler
  // then knows that a copy into one buffer does not write another, and
  // inserts no wait for the copies before reading a different buffer.
  __shared__ __attribute__((aligned(1024))) uint8_t lds_q0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_q1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_q2[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_g0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_g1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_g2[TILEB];
  // LSE (copied by wave 0) and D (wave 1) of the tile's queries: one 256-byte
  // copy each, of which the first 128 bytes are the 32 values
  __shared__ __attribute__((aligned(256))) float lds_l0[64];
  __shared__ __attribute__((aligned(256))) float lds_l1[64];
  __shared__ __attribute__((aligned(256))) float lds_l2[64];
  __shared__ __attribute__((aligned(256))) float lds_d0[64];
  __shared__ __attribute__((aligned(256))) float lds_d1[64];
  __shared__ __attribute__((aligned(256))) float lds_d2[64];
  // buffer i (compile-time) of each kind
  auto bq = [&](auto it) __attribute__((always_inline)) -> uint8_t* {
    constexpr int i = decltype(it)::value;
    return i == 0 ? lds_q0 : i == 1 ? lds_q1 : lds_q2;
  };
  auto bg = [&](auto it) __attribute__((always_inline)) -> uint8_t* {
    constexpr int i = decltype(it)::value;
    return i == 0 ? lds_g0 : i == 1 ? lds_g1 : lds_g2;
  };
  auto bl = [&](auto it) __attribute__((always_inline)) -> float* {
    constexpr int i = decltype(it)::value;
    return i == 0 ? lds_l0 : i == 1 ? lds_l1 : lds_l2;
  };
  auto bd = [&](auto it) __attribute__((always_inline)) -> float* {
    constexpr int i = decltype(it)::value;
    return i == 0 ? lds_d0 : i == 1 ? lds_d1 : lds_d2;
  };

  // work item: (batch, head, key block), a head's blocks on one XCD
  const int lin = blockIdx.x;
  const int BH = p.B * p.H;
  const bool by_xcd = (BH & 7) == 0;
  const int nh = by_xcd ? BH >> 3 : BH;
  // one (d = 128) or two (d = 64) workgroups per CU
  const int kk = by_xcd ? engine_order(lin >> 3, nh * p.n_tiles, D == 128 ? 32 : 64) : lin;
  const int ki = kk / nh;
  const int hh = kk - ki * nh;
  const int bh = by_xcd ? 8 * hh + (lin & 7) : hh;
  const int kt = ki;  // key block; causal: later blocks see fewer queries
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int k0 = kt * kBKV;

  const size_t rs = (size_t)p.H * D;
  const size_t qo = ((size_t)b * p.Nq * p.H + h) * D;
  const size_t kvo = ((size_t)b * p.Nk * p.H + h) * D;
  const uint32_t row_bytes = (uint32_t)(rs * 2);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int kw0 = k0 + wave * 32;
  const int my_k = kw0 + ln;

  // K and -V fragments of this wave's keys (B operands), read once
  u32x4 kf[DK], vf[DK];
  if (my_k < p.Nk) {
    const uint16_t* krow = p.k + kvo + (size_t)my_k * rs + 8 * hf;
    const uint16_t* vrow = p.v + kvo + (size_t)my_k * rs + 8 * hf;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      kf[i] = *reinterpret_cast<const u32x4*>(krow + 16 * i);
      vf[i] = *reinterpret_cast<const u32x4*>(vrow + 16 * i);
      // negated (sign bits flipped, exact): the dP MFMAs then compute D - dP
#pragma unroll
      for (int w = 0; w < 4; ++w) vf[i][w] ^= 0x80008000u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < DK; ++i) kf[i] = vf[i] = u32x4{0, 0, 0, 0};
  }

  // query tiles: causal blocks start at the first query that sees key k0
  const int n_qtiles_all = (p.Nq + BQt - 1) / BQt;
  const int t_begin = CAUSAL ? min(k0 / BQt, n_qtiles_all) : 0;

  uint32_t c_off[NCPW];
#pragma unroll
  for (int c = 0; c < NCPW; ++c) {
    const int row = (c * NW + wave) * RPI + lane / CH;
    c_off[c] = row * row_bytes + 16 * ((lane % CH) ^ bwd::t_swz<D>(row));
  }
  // copies per wave per tile: NCPW each of Q and dO, plus LSE on wave 0 and
  // D on wave 1 (their rows of this (b, h), chosen once)
  const float* const lsd_src = (wave == 0 ? p.lse : p.delta) + (size_t)bh * p.Nq;
  auto issue = [&](int t, uint8_t* lq, uint8_t* lg, float* ll, float* ld) __attribute__((always_inline)) {
    const int nvalid = min(BQt, p.Nq - t * BQt);
    const uint32_t bytes = (uint32_t)(nvalid - 1) * row_bytes + ROWB;
    const auto rq = make_rsrc(p.q + qo + (size_t)t * BQt * rs, bytes);
    const auto rg = make_rsrc(p.dout + qo + (size_t)t * BQt * rs, bytes);
#pragma unroll
    for (int c = 0; c < NCPW; ++c) dma16(rq, lq + (c * NW + wave) * 1024, c_off[c]);
#pragma unroll
    for (int c = 0; c < NCPW; ++c) dma16(rg, lg + (c * NW + wave) * 1024, c_off[c]);
    if (wave < 2) {
      const auto rl = make_rsrc(lsd_src + t * BQt, (uint32_t)nvalid * 4);
      bwd::dma4(rl, reinterpret_cast<uint8_t*>(wave == 0 ? ll : ld), 4 * lane);
    }
  };

  uint32_t roff[DK];
  {
    const int row = k_row_order(ln);
    const int sw = bwd::t_swz<D>(row);
#pragma unroll
    for (int i = 0; i < DK; ++i) roff[i] = row * ROWB + 16 * ((2 * i + hf) ^ sw);
  }
  uint32_t toff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 2; ++r) toff[db][r] = bwd::tr_off<D>(lane, db, r);

  f32x16 dkt[DB], dvt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkt[db][r] = dvt[db][r] = 0.f;
  const float c = p.scale_log2;

  // One query tile: 4 MFMA phases, 32 MFMAs at d = 128, run as one sequence
  // of fenced slots. Slot j holds MFMA j, the LDS read of the operand of
  // MFMA j + kA (one operand ring across all phases and on into the next
  // tile) and a share of the VALU work, spread so that no slot holds much
  // more than the MFMA covers (one wave per SIMD at d = 128: no other wave
  // would hide it):
  //   1. S = Q K^T                (N1 MFMAs)   VALU: -LSE log2 e
  //   2. dP' = D - dO V^T         (N2 MFMAs)   VALU: P = exp2(S c - LSE log2 e),
  //   3. dV^T += dO^T P           (N3 MFMAs)         spread over 2 and half of 3
  //   4. -dK^T += Q^T (P o dP')   (N4 MFMAs)   VALU: -dS = P o dP', spread over
  //                                                  the rest of 3 and half of 4
  // dP' starts from D (the accumulator input of its first MFMA) and takes
  // the negated V fragments, so -dS is one product per element; the sign
  // comes back when dK is stored. Operands: Q rows and dO rows (phases 1,
  // 2) by row reads of the swizzled tiles, dO^T and Q^T (phases 3, 4) by
  // transpose reads. The tiles are triple-buffered, so the next tile is
  // complete while this one runs: the last slots read its LSE and D, the ring
  // carries its first kA operands, and its first MFMA does not wait for LDS
  // after the barrier.
  // The slots are generated at compile time (static_for, if constexpr), so
  // the code of each is straight-line from the start: with a run-time slot
  // index the optimiser moved MFMAs of the rolled loop several slots late.
  // The asm statements on the values computed in a slot keep the compiler
  // from sinking that arithmetic to its use in a later slot. Each holds one
  // s_nop: the compiler counts every asm statement as one wait state when it
  // spaces an MFMA and a VALU read of its result, so an empty one would
  // leave such a read a wait state short.
  constexpr int N1 = DK, N2 = DK, N3 = PK * DB, N4 = PK * DB;
  constexpr int NM = N1 + N2 + N3 + N4;
  constexpr int kA = bwd::kDkdvAhead;
  static_assert(NM - kA - 2 * PK >= N1, "next-tile LSE/D reads after phase 1");
  // operand of MFMA j of the tile in (lq, lg)
  auto operand = [&](auto jt, const uint8_t* lq, const uint8_t* lg) __attribute__((always_inline)) -> u32x4 {
    constexpr int j = decltype(jt)::value;
    if constexpr (j < N1) {
      return *reinterpret_cast<const u32x4*>(lq + roff[j]);
    } else if constexpr (j < N1 + N2) {
      return *reinterpret_cast<const u32x4*>(lg + roff[j - N1]);
    } else {
      constexpr bool dv_phase = j < N1 + N2 + N3;
      constexpr int m = dv_phase ? j - N1 - N2 : j - N1 - N2 - N3;
      return bwd::tr_operand((dv_phase ? lg : lq) + (m / DB) * 16 * ROWB, toff[m % DB][0],
                             toff[m % DB][1]);
    }
  };
  // LSE and D of this lane's 16 queries (element r is query
  // qt0 + 16*(r>>3) + 8*hf + (r&7)), half i of the reads
  u32x4 lq4[2 * PK], dq4[2 * PK], ring[kA];
  auto read_ld = [&](auto it, const float* ll, const float* ld) __attribute__((always_inline)) {
    constexpr int i = decltype(it)::value;
    const int qr = 16 * (i >> 1) + 8 * hf + 4 * (i & 1);
    lq4[i] = *reinterpret_cast<const u32x4*>(ll + qr);
    dq4[i] = *reinterpret_cast<const u32x4*>(ld + qr);
  };
  // what a tile needs read before its first slot
  auto prefetch = [&](const uint8_t* lq, const uint8_t* lg, const float* ll, const float* ld)
                      __attribute__((always_inline)) {
    bwd::static_for<0, 2 * PK>([&](auto it) __attribute__((always_inline)) { read_ld(it, ll, ld); });
    bwd::static_for<0, kA>([&](auto jt) __attribute__((always_inline)) {
      ring[decltype(jt)::value] = operand(jt, lq, lg);
    });
  };
  auto tile_body = [&](int t, const uint8_t* lq, const uint8_t* lg, auto mask_tag, auto&& next,
                       const uint8_t* nq, const uint8_t* ng, const float* nll, const float* nld)
                       __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int EP1 = 16 / N1;  // -LSE log2 e values per phase-1 slot
    static_assert(EP1 % 2 == 0, "pairs per slot");
    // P over the N2 + N3/2 - 1 slots from N1 on, each half done before the
    // dV MFMAs that take it; -dS over the slots after, up to the middle of
    // phase 4, each half done before the dK MFMAs that take it
    using SpreadP = bwd::Spread<N1, N2 + N3 / 2 - 1>;
    using SpreadD = bwd::Spread<N1 + N2 + N3 / 2 - 1, N3 / 2 + N4 / 2 + 1>;
    static_assert(SpreadP::lo(N1 + N2) >= 8 && SpreadP::lo(N1 + N2 + N3 / 2) == 16, "P in time");
    static_assert(SpreadD::lo(N1 + N2 + N3) >= 8 && SpreadD::lo(N1 + N2 + N3 + N4 / 2) == 16,
                  "dS in time");
    // the next tile's LSE and D are read from slot kLd on (this tile's are
    // dead by then: phase 1 and the seeding of dP' use them)
    constexpr int kLd = NM - kA - 2 * PK;
    const int qt0 = t * BQt;
    const bwd::QueryMask<CAUSAL> qmask(qt0, hf, my_k, p.Nq);

    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // (read as plain integers first: __builtin_bit_cast of a vector
      // element reads element 0)
      const uint32_t b = dq4[r >> 2][r & 3];
      s[r] = 0.f;
      dp[r] = __builtin_bit_cast(float, b);
    }
    float nl[16], pr[16], nds[16];
    u32x4 pp[PK], dsp[PK];
    bwd::static_for<0, NM>([&](auto jt) __attribute__((always_inline)) {
      constexpr int j = decltype(jt)::value;
      const u32x4 a = ring[j % kA];
      if constexpr (j + kA < NM) ring[j % kA] = operand(std::integral_constant<int, j + kA>{}, lq, lg);
      else ring[j % kA] = operand(std::integral_constant<int, j + kA - NM>{}, nq, ng);
      if constexpr (j >= kLd && j < kLd + 2 * PK)
        read_ld(std::integral_constant<int, j - kLd>{}, nll, nld);
      if constexpr (j < N1) {
        s = O_::mfma(a, kf[j], s);
        if constexpr (j == 0) next();  // the tile after next: copies into the free buffer
      } else if constexpr (j < N1 + N2) {
        dp = O_::mfma(a, vf[j - N1], dp);
      } else if constexpr (j < N1 + N2 + N3) {
        constexpr int m = j - N1 - N2;
        dvt[m % DB] = O_::mfma(a, pp[m / DB], dvt[m % DB]);
      } else {
        constexpr int m = j - N1 - N2 - N3;
        dkt[m % DB] = O_::mfma(a, dsp[m / DB], dkt[m % DB]);
      }
      // exponent offsets of elements [j*EP1, (j+1)*EP1)
      if constexpr (j < N1) {
        bwd::static_for<0, EP1 / 2>([&](auto it) __attribute__((always_inline)) {
          constexpr int r = j * EP1 + 2 * decltype(it)::value;
          const uint32_t b0 = lq4[r >> 2][r & 3], b1 = lq4[(r + 1) >> 2][(r + 1) & 3];
          float x0 = __builtin_bit_cast(float, b0) * -bwd::kLog2e;
          float x1 = __builtin_bit_cast(float, b1) * -bwd::kLog2e;
          asm volatile("s_nop 0" : "+v"(x0), "+v"(x1));
          nl[r] = x0;
          nl[r + 1] = x1;
        });
      }
      // P of elements [SpreadP::lo(j), SpreadP::lo(j + 1)), packed in pairs
      bwd::static_for<SpreadP::lo(j), SpreadP::lo(j + 1)>([&](auto rt) __attribute__((always_inline)) {
        constexpr int r = decltype(rt)::value;
        float x = fast_exp2(__builtin_fmaf(s[r], c, nl[r]));
        if constexpr (MASK) x = qmask.visible(16 * (r >> 3) + (r & 7)) ? x : 0.f;
        if constexpr (r & 1) {
          uint32_t w = O_::pack(pr[r - 1], x);
          asm volatile("s_nop 0" : "+v"(w));
          pp[r >> 3][(r & 7) >> 1] = w;
        } else if constexpr (r + 1 == SpreadP::lo(j + 1)) {
          asm volatile("s_nop 0" : "+v"(x));  // its pair is packed in a later slot
        }
        pr[r] = x;
      });
      // -dS of elements [SpreadD::lo(j), SpreadD::lo(j + 1)), packed in pairs
      bwd::static_for<SpreadD::lo(j), SpreadD::lo(j + 1)>([&](auto rt) __attribute__((always_inline)) {
        constexpr int r = decltype(rt)::value;
        float y = pr[r] * dp[r];
        if constexpr (r & 1) {
          uint32_t w = O_::pack(nds[r - 1], y);
          asm volatile("s_nop 0" : "+v"(w));
          dsp[r >> 3][(r & 7) >> 1] = w;
        } else if constexpr (r + 1 == SpreadD::lo(j + 1)) {
          asm volatile("s_nop 0" : "+v"(y));
        }
        nds[r] = y;
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // Steps: one per query tile u = 0 .. n_t-1 (tile t_begin + u), each with
  // one barrier; tile u lives in buffer u % 3. At the barrier of step u the
  // copies of tile u + 1 (issued in step u - 1) are complete and every wave
  // is done with tile u - 1, whose buffer then takes tile u + 2. A causal
  // wave has nothing to do for its first `f` tiles (all their queries
  // precede its keys); tile f is its diagonal tile (the only one that needs
  // an element mask, as BQt = 32 keys per wave); the rest are fully
  // visible. Rows past Nq need no mask: their Q, dO, LSE and D are
  // zero-filled, so P = 1 and dS = 0 multiply zero rows. Each kind of step
  // is a straight-line body with the buffer index fixed at compile time, so
  // the accumulators stay in place. The last step reads a stale buffer as
  // its next tile (in bounds, never used).
  const int n_t = n_qtiles_all - t_begin;
  int f = CAUSAL ? min(n_t, wave) : 0;
  if (kw0 >= p.Nk) f = n_t;  // no real keys in this wave
  auto step = [&](int u, auto par, auto mode) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    constexpr int P1 = (P + 1) % 3, P2 = (P + 2) % 3;
    constexpr int MODE = decltype(mode)::value;  // 0 idle, 1 masked, 2 unmasked
    const int t = t_begin + u;
    // vmcnt(0): this wave's copies of tile u + 1 are done. lgkmcnt(kA): all
    // but its last kA LDS reads are done; those are the ring reads of tile
    // u + 1 (LDS reads complete in order), and what the barrier frees is
    // tile u - 1's buffer
    static_assert(kA < 16, "lgkmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0070 | (kA << 8));
    sync::bare_barrier();
    using I = std::integral_constant<int, P>;
    using I1 = std::integral_constant<int, P1>;
    using I2 = std::integral_constant<int, P2>;
    auto next = [&]() __attribute__((always_inline)) {
      if (u + 2 < n_t) issue(t + 2, bq(I2{}), bg(I2{}), bl(I2{}), bd(I2{}));
    };
    if constexpr (MODE != 0) {
      using M = std::integral_constant<bool, MODE == 1>;
      tile_body(t, bq(I{}), bg(I{}), M{}, next, bq(I1{}), bg(I1{}), bl(I1{}), bd(I1{}));
    } else {
      next();
      prefetch(bq(I1{}), bg(I1{}), bl(I1{}), bd(I1{}));
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  auto run = [&](int u0, int u1, auto mode) __attribute__((always_inline)) {
    int u = u0;
    if (u < u1 && u % 3 == 1) step(u++, B1{}, mode);
    if (u < u1 && u % 3 == 2) step(u++, B2{}, mode);
    for (; u + 2 < u1; u += 3) {
      step(u, B0{}, mode);
      step(u + 1, B1{}, mode);
      step(u + 2, B2{}, mode);
    }
    if (u < u1) step(u++, B0{}, mode);
    if (u < u1) step(u, B1{}, mode);
  };
  // prologue: tile 0 complete and visible, tile 1 in flight, tile 0's
  // first reads issued
  if (n_t > 0) issue(t_begin, lds_q0, lds_g0, lds_l0, lds_d0);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
  if (n_t > 1) issue(t_begin + 1, lds_q1, lds_g1, lds_l1, lds_d1);
  sync::bare_barrier();
  prefetch(lds_q0, lds_g0, lds_l0, lds_d0);
  run(0, f, std::integral_constant<int, 0>{});
  if constexpr (CAUSAL) {
    if (f < n_t) {
      const int fb = f % 3;
      if (fb == 0) step(f, B0{}, std::integral_constant<int, 1>{});
      else if (fb == 1) step(f, B1{}, std::integral_constant<int, 1>{});
      else step(f, B2{}, std::integral_constant<int, 1>{});
    }
  }
  run(f + (CAUSAL ? 1 : 0), n_t, std::integral_constant<int, 2>{});

  // dK = scale * dK^T, dV = dV^T (lane = key, registers = head-dim index),
  // stored as whole rows through one Q/dO tile buffer per wave (free once
  // every wave has left the tile loop; no copy is in flight)
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
  sync::bare_barrier();
  {
    const int nrows = min(kBKV, p.Nk - k0);
    const uint32_t range = (uint32_t)(nrows - 1) * row_bytes + 2 * D;
    const auto out_k = make_rsrc(p.dk + kvo + (size_t)k0 * rs, range);
    const auto out_v = make_rsrc(p.dv + kvo + (size_t)k0 * rs, range);
    uint8_t* const slot = wave == 0 ? lds_q0 : wave == 1 ? lds_q1 : wave == 2 ? lds_q2 : lds_g0;
    const uint32_t gbase = (uint32_t)(wave * 32) * row_bytes;
    store_rows<O_, D>(dkt, -p.scale, slot, out_k, gbase, row_bytes, lane);  // dkt holds -dK^T
    store_rows<O_, D>(dvt, 1.f, slot, out_v, gbase, row_bytes, lane);
  }
}

// ---- dK, dV at d = 128: producer/consumer wave pairs -----------------------
// The kernel above runs one wave per SIMD at d = 128 (~330 registers), and a
// lone wave draws only ~1 KiB per 29 cycles from LDS with 16-byte reads: its
// tile is bound by its own LDS reads, not by the MFMA pipe. Here each SIMD
// runs two waves of one workgroup on the same 32 keys:
// * a producer (waves 0-3) holds the K and -V fragments and, for query tile
//   u, computes S = Q K^T and dP' = D - dO V^T (16 MFMAs) with -LSE log2 e,
//   P and -dS = P o dP' between and after them, and hands P and -dS (packed,
//   the MFMA B-operand fragments, 4 KiB per wave) to its consumer through
//   LDS;
// * the consumer (waves 4-7, on the same SIMD, same keys) holds dV^T and
//   -dK^T and, in the same step, accumulates dV^T += dO^T P and
//   -dK^T += Q^T (-dS) for tile u - 1 (16 MFMAs, the transpose reads).
// Each wave holds about half of the state, so both fit 256 registers, and
// each issues about half of a tile's LDS reads; the MFMA pipe of the SIMD
// takes both waves' MFMAs. One barrier per step orders the hand-over (step
// u's producers write exchange buffer u % 2, step u + 1's consumers read
// it). Q/dO tiles rotate through four buffers (tile u - 1 is still read by
// the consumers while tile u + 2 is copied in); the consumers issue the
// copies. The arithmetic and its order per element are those of the kernel
// above, so the results are identical to it.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(2 * bwd::kThreads) void mha_bwd_dkdv_pair_kernel(BwdParams p) {
  using O_ = Ops<T>;
  constexpr int BQt = bwd::kBQt;
  constexpr int kBKV = bwd::kBKV;
  constexpr int NP = bwd::kWaves;          // wave pairs, 32 keys each
  constexpr int DK = D / 16;
  constexpr int DB = D / 32;
  constexpr int PK = BQt / 16;
  constexpr int CH = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BQt * ROWB;        // Q or dO tile
  constexpr int RPI = 1024 / ROWB;
  constexpr int NCPW = TILEB / 1024 / NP;  // copies per consumer wave per tensor
  constexpr int XB = 2 * PK * 1024;        // exchange bytes per pair: P and -dS, 16 B per lane each
  static_assert(NCPW >= 1 && (NP * RPI) % 16 == 0, "copy layout");
  constexpr int kA = bwd::kDkdvAhead;
  constexpr int NMP = 2 * DK;              // producer MFMAs per tile
  constexpr int NMC = 2 * PK * DB;         // consumer MFMAs per tile

  // Four buffers of each tile kind, two exchange buffers; separate objects,
  // so that the compiler sees that a copy into one buffer does not write
  // another and inserts no wait for the copies before other LDS reads.
  __shared__ __attribute__((aligned(1024))) uint8_t lds_q0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_q1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_q2[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_q3[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_g0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_g1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_g2[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_g3[TILEB];
  // LSE (copied by pair 0's consumer) and D (pair 1's) of the tile's
  // queries: one 256-byte copy each, of which the first 128 bytes are the 32
  // values
  __shared__ __attribute__((aligned(256))) float lds_l0[64];
  __shared__ __attribute__((aligned(256))) float lds_l1[64];
  __shared__ __attribute__((aligned(256))) float lds_l2[64];
  __shared__ __attribute__((aligned(256))) float lds_l3[64];
  __shared__ __attribute__((aligned(256))) float lds_d0[64];
  __shared__ __attribute__((aligned(256))) float lds_d1[64];
  __shared__ __attribute__((aligned(256))) float lds_d2[64];
  __shared__ __attribute__((aligned(256))) float lds_d3[64];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_x0[NP * XB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_x1[NP * XB];
  // buffer i (compile-time) of each kind
  auto bq = [&](auto it) __attribute__((always_inline)) -> uint8_t* {
    constexpr int i = decltype(it)::value & 3;
    return i == 0 ? lds_q0 : i == 1 ? lds_q1 : i == 2 ? lds_q2 : lds_q3;
  };
  auto bg = [&](auto it) __attribute__((always_inline)) -> uint8_t* {
    constexpr int i = decltype(it)::value & 3;
    return i == 0 ? lds_g0 : i == 1 ? lds_g1 : i == 2 ? lds_g2 : lds_g3;
  };
  auto bl = [&](auto it) __attribute__((always_inline)) -> float* {
    constexpr int i = decltype(it)::value & 3;
    return i == 0 ? lds_l0 : i == 1 ? lds_l1 : i == 2 ? lds_l2 : lds_l3;
  };
  auto bd = [&](auto it) __attribute__((always_inline)) -> float* {
    constexpr int i = decltype(it)::value & 3;
    return i == 0 ? lds_d0 : i == 1 ? lds_d1 : i == 2 ? lds_d2 : lds_d3;
  };
  auto bx = [&](auto it) __attribute__((always_inline)) -> uint8_t* {
    return (decltype(it)::value & 1) == 0 ? lds_x0 : lds_x1;
  };

  // work item: (batch, head, key block), a head's blocks on one XCD, one
  // workgroup per CU
  const int lin = blockIdx.x;
  const int BH = p.B * p.H;
  const bool by_xcd = (BH & 7) == 0;
  const int nh = by_xcd ? BH >> 3 : BH;
  const int kk = by_xcd ? engine_order(lin >> 3, nh * p.n_tiles, 32) : lin;
  const int ki = kk / nh;
  const int hh = kk - ki * nh;
  const int bh = by_xcd ? 8 * hh + (lin & 7) : hh;
  const int kt = ki;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int k0 = kt * kBKV;

  const size_t rs = (size_t)p.H * D;
  const size_t qo = ((size_t)b * p.Nq * p.H + h) * D;
  const size_t kvo = ((size_t)b * p.Nk * p.H + h) * D;
  const uint32_t row_bytes = (uint32_t)(rs * 2);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & (NP - 1);
  const bool consumer = wave >= NP;
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int kw0 = k0 + pair * 32;
  const int my_k = kw0 + ln;

  // query tiles: causal blocks start at the first query that sees key k0
  const int n_qtiles_all = (p.Nq + BQt - 1) / BQt;
  const int t_begin = CAUSAL ? min(k0 / BQt, n_qtiles_all) : 0;
  const int n_t = n_qtiles_all - t_begin;
  // a causal pair has nothing to do for its first f tiles; tile f is its
  // diagonal tile (element mask), the rest are fully visible (rows past Nq:
  // zero-filled Q, dO, LSE and D, so P = 1 and dS = 0 on zero rows)
  int f = CAUSAL ? min(n_t, pair) : 0;
  if (kw0 >= p.Nk) f = n_t;  // no real keys in this pair

  uint32_t roff[DK];
  {
    const int row = k_row_order(ln);
    const int sw = bwd::t_swz<D>(row);
#pragma unroll
    for (int i = 0; i < DK; ++i) roff[i] = row * ROWB + 16 * ((2 * i + hf) ^ sw);
  }
  uint32_t toff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 2; ++r) toff[db][r] = bwd::tr_off<D>(lane, db, r);
  // this lane's 16 bytes of a pair's exchange block
  const uint32_t xoff = (uint32_t)(pair * XB + 16 * lane);

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;
  // steps u0 .. u1-1 of one kind, tile buffers u % 4 fixed at compile time
  auto run4 = [&](int u0, int u1, auto&& step) __attribute__((always_inline)) {
    int u = u0;
    if (u < u1 && (u & 3) == 1) step(u++, B1{});
    if (u < u1 && (u & 3) == 2) step(u++, B2{});
    if (u < u1 && (u & 3) == 3) step(u++, B3{});
    for (; u + 3 < u1; u += 4) {
      step(u, B0{});
      step(u + 1, B1{});
      step(u + 2, B2{});
      step(u + 3, B3{});
    }
    if (u < u1) step(u++, B0{});
    if (u < u1) step(u++, B1{});
    if (u < u1) step(u, B2{});
  };
  auto at4 = [&](int u, auto&& step) __attribute__((always_inline)) {
    switch (u & 3) {
      case 0: step(u, B0{}); break;
      case 1: step(u, B1{}); break;
      case 2: step(u, B2{}); break;
      default: step(u, B3{}); break;
    }
  };

  // copies per consumer wave per tile: NCPW each of Q and dO, plus LSE on
  // pair 0 and D on pair 1 (their rows of this (b, h), chosen once)
  uint32_t c_off[NCPW];
#pragma unroll
  for (int c = 0; c < NCPW; ++c) {
    const int row = (c * NP + pair) * RPI + lane / CH;
    c_off[c] = row * row_bytes + 16 * ((lane % CH) ^ bwd::t_swz<D>(row));
  }
  const float* const lsd_src = (pair == 0 ? p.lse : p.delta) + (size_t)bh * p.Nq;
  auto issue = [&](int t, uint8_t* lq, uint8_t* lg, float* ll, float* ld) __attribute__((always_inline)) {
    const int nvalid = min(BQt, p.Nq - t * BQt);
    const uint32_t bytes = (uint32_t)(nvalid - 1) * row_bytes + ROWB;
    const auto rq = make_rsrc(p.q + qo + (size_t)t * BQt * rs, bytes);
    const auto rg = make_rsrc(p.dout + qo + (size_t)t * BQt * rs, bytes);
#pragma unroll
    for (int c = 0; c < NCPW; ++c) dma16(rq, lq + (c * NP + pair) * 1024, c_off[c]);
#pragma unroll
    for (int c = 0; c < NCPW; ++c) dma16(rg, lg + (c * NP + pair) * 1024, c_off[c]);
    if (pair < 2) {
      const auto rl = make_rsrc(lsd_src + t * BQt, (uint32_t)nvalid * 4);
      bwd::dma4(rl, reinterpret_cast<uint8_t*>(pair == 0 ? ll : ld), 4 * lane);
    }
  };

  const float c = p.scale_log2;

  if (!consumer) {
    // ---------------------------------------------------------- producer
    // K and -V fragments of this pair's keys (B operands), read once
    u32x4 kf[DK], vf[DK];
    if (my_k < p.Nk) {
      const uint16_t* krow = p.k + kvo + (size_t)my_k * rs + 8 * hf;
      const uint16_t* vrow = p.v + kvo + (size_t)my_k * rs + 8 * hf;
#pragma unroll
      for (int i = 0; i < DK; ++i) {
        kf[i] = *reinterpret_cast<const u32x4*>(krow + 16 * i);
        vf[i] = *reinterpret_cast<const u32x4*>(vrow + 16 * i);
        // negated (sign bits flipped, exact): the dP MFMAs then compute D - dP
#pragma unroll
        for (int w = 0; w < 4; ++w) vf[i][w] ^= 0x80008000u;
      }
    } else {
#pragma unroll
      for (int i = 0; i < DK; ++i) kf[i] = vf[i] = u32x4{0, 0, 0, 0};
    }
    // operand of MFMA j (row reads: Q rows for S, dO rows for dP)
    auto operand = [&](auto jt, const uint8_t* lq, const uint8_t* lg) __attribute__((always_inline)) -> u32x4 {
      constexpr int j = decltype(jt)::value;
      if constexpr (j < DK) return *reinterpret_cast<const u32x4*>(lq + roff[j]);
      else return *reinterpret_cast<const u32x4*>(lg + roff[j - DK]);
    };
    // LSE and D of this lane's 16 queries (element r is query
    // t*BQt + 16*(r>>3) + 8*hf + (r&7)), half i of the reads
    u32x4 lq4[2 * PK], dq4[2 * PK], ring[kA];
    auto read_ld = [&](auto it, const float* ll, const float* ld) __attribute__((always_inline)) {
      constexpr int i = decltype(it)::value;
      const int qr = 16 * (i >> 1) + 8 * hf + 4 * (i & 1);
      lq4[i] = *reinterpret_cast<const u32x4*>(ll + qr);
      dq4[i] = *reinterpret_cast<const u32x4*>(ld + qr);
    };
    // what a tile needs read before its first slot
    auto prefetch = [&](const uint8_t* lq, const uint8_t* lg, const float* ll, const float* ld)
                        __attribute__((always_inline)) {
      bwd::static_for<0, 2 * PK>([&](auto it) __attribute__((always_inline)) { read_ld(it, ll, ld); });
      bwd::static_for<0, kA>([&](auto jt) __attribute__((always_inline)) {
        ring[decltype(jt)::value] = operand(jt, lq, lg);
      });
    };
    // One query tile: 2*DK fenced slots (S, then dP'), each with one MFMA,
    // the operand read kA MFMAs ahead (on into the next tile) and a share of
    // the VALU work: -LSE log2 e in the S slots, P in the dP' slots; -dS after
    // them; then P and -dS to the exchange block. The next tile's LSE and D
    // are read from slot kLd on (this tile's are used by then).
    constexpr int kLd = NMP - kA - 2 * PK;
    static_assert(kLd >= DK, "next-tile LSE/D reads after the S slots");
    constexpr int EP = 16 / DK;  // elements per slot (-LSE log2 e, P)
    static_assert(EP % 2 == 0, "pairs per slot");
    auto tile = [&](int t, const uint8_t* lq, const uint8_t* lg, auto mask_tag, const uint8_t* nq,
                    const uint8_t* ng, const float* nll, const float* nld, uint8_t* xb)
                    __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int qt0 = t * BQt;
      const bwd::QueryMask<CAUSAL> qmask(qt0, hf, my_k, p.Nq);
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // (read as plain integers first: __builtin_bit_cast of a vector
        // element reads element 0)
        const uint32_t bb = dq4[r >> 2][r & 3];
        s[r] = 0.f;
        dp[r] = __builtin_bit_cast(float, bb);
      }
      float nl[16], pr[16];
      u32x4 pp[PK], dsp[PK];
      bwd::static_for<0, NMP>([&](auto jt) __attribute__((always_inline)) {
        constexpr int j = decltype(jt)::value;
        const u32x4 a = ring[j % kA];
        if constexpr (j + kA < NMP) ring[j % kA] = operand(std::integral_constant<int, j + kA>{}, lq, lg);
        else ring[j % kA] = operand(std::integral_constant<int, j + kA - NMP>{}, nq, ng);
        if constexpr (j >= kLd && j < kLd + 2 * PK)
          read_ld(std::integral_constant<int, j - kLd>{}, nll, nld);
        if constexpr (j < DK) {
          s = O_::mfma(a, kf[j], s);
          bwd::static_for<0, EP / 2>([&](auto it) __attribute__((always_inline)) {
            constexpr int r = j * EP + 2 * decltype(it)::value;
            const uint32_t b0 = lq4[r >> 2][r & 3], b1 = lq4[(r + 1) >> 2][(r + 1) & 3];
            float x0 = __builtin_bit_cast(float, b0) * -bwd::kLog2e;
            float x1 = __builtin_bit_cast(float, b1) * -bwd::kLog2e;
            asm volatile("s_nop 0" : "+v"(x0), "+v"(x1));
            nl[r] = x0;
            nl[r + 1] = x1;
          });
        } else {
          dp = O_::mfma(a, vf[j - DK], dp);
          bwd::static_for<0, EP / 2>([&](auto it) __attribute__((always_inline)) {
            constexpr int r = (j - DK) * EP + 2 * decltype(it)::value;
            float x[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              x[e] = fast_exp2(__builtin_fmaf(s[r + e], c, nl[r + e]));
              if constexpr (MASK) x[e] = qmask.visible(16 * ((r + e) >> 3) + ((r + e) & 7)) ? x[e] : 0.f;
              pr[r + e] = x[e];
            }
            uint32_t w = O_::pack(x[0], x[1]);
            asm volatile("s_nop 0" : "+v"(w));
            pp[r >> 3][(r & 7) >> 1] = w;
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      // -dS = P o dP' (dP' = D - dP), packed
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        dsp[r >> 3][(r & 7) >> 1] = O_::pack(pr[r] * dp[r], pr[r + 1] * dp[r + 1]);
#pragma unroll
      for (int ks = 0; ks < PK; ++ks) {
        *reinterpret_cast<u32x4*>(xb + xoff + ks * 1024) = pp[ks];
        *reinterpret_cast<u32x4*>(xb + xoff + (PK + ks) * 1024) = dsp[ks];
      }
    };
    // step u: tile u, exchange buffer u % 2
    auto step_of = [&](auto mode) __attribute__((always_inline)) {
      return [&, mode](int u, auto par) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        constexpr int MODE = decltype(mode)::value;  // 0 idle, 1 masked, 2 unmasked
        using I = std::integral_constant<int, P>;
        using I1 = std::integral_constant<int, P + 1>;
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0): exchange writes done
        sync::bare_barrier();
        if constexpr (MODE != 0) {
          using M = std::integral_constant<bool, MODE == 1>;
          tile(t_begin + u, bq(I{}), bg(I{}), M{}, bq(I1{}), bg(I1{}), bl(I1{}), bd(I1{}), bx(I{}));
        } else {
          prefetch(bq(I1{}), bg(I1{}), bl(I1{}), bd(I1{}));
        }
      };
    };
    // prologue (the consumers copy tiles 0 and 1): tile 0's first reads
    sync::bare_barrier();
    prefetch(lds_q0, lds_g0, lds_l0, lds_d0);
    run4(0, f, step_of(std::integral_constant<int, 0>{}));
    if constexpr (CAUSAL) {
      if (f < n_t) at4(f, step_of(std::integral_constant<int, 1>{}));
    }
    run4(f + (CAUSAL ? 1 : 0), n_t, step_of(std::integral_constant<int, 2>{}));
    // the consumers' last step (tile n_t - 1)
    __builtin_amdgcn_s_waitcnt(0x0070);
    sync::bare_barrier();
    // epilogue: the consumers store
    __builtin_amdgcn_s_waitcnt(0x0070);
    sync::bare_barrier();
  } else {
    // ---------------------------------------------------------- consumer
    f32x16 dkt[DB], dvt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dkt[db][r] = dvt[db][r] = 0.f;
    // operand of MFMA j: dO^T (dV phase) or Q^T (dK phase) by transpose reads
    auto operand = [&](auto jt, const uint8_t* lq, const uint8_t* lg) __attribute__((always_inline)) -> u32x4 {
      constexpr int j = decltype(jt)::value;
      constexpr bool dv_phase = j < PK * DB;
      constexpr int m = dv_phase ? j : j - PK * DB;
      return bwd::tr_operand((dv_phase ? lg : lq) + (m / DB) * 16 * ROWB, toff[m % DB][0],
                             toff[m % DB][1]);
    };
    u32x4 ring[kA];
    auto prefetch = [&](const uint8_t* lq, const uint8_t* lg) __attribute__((always_inline)) {
      bwd::static_for<0, kA>([&](auto jt) __attribute__((always_inline)) {
        ring[decltype(jt)::value] = operand(jt, lq, lg);
      });
    };
    // tile u - 1: P and -dS from the exchange block, then 2*PK*DB fenced
    // slots (dV^T, then -dK^T), the operand read kA MFMAs ahead (on into
    // tile u)
    auto tile = [&](const uint8_t* lq, const uint8_t* lg, const uint8_t* xb, const uint8_t* nq,
                    const uint8_t* ng) __attribute__((always_inline)) {
      u32x4 pp[PK], dsp[PK];
#pragma unroll
      for (int ks = 0; ks < PK; ++ks) {
        pp[ks] = *reinterpret_cast<const u32x4*>(xb + xoff + ks * 1024);
        dsp[ks] = *reinterpret_cast<const u32x4*>(xb + xoff + (PK + ks) * 1024);
      }
      bwd::static_for<0, NMC>([&](auto jt) __attribute__((always_inline)) {
        constexpr int j = decltype(jt)::value;
        const u32x4 a = ring[j % kA];
        if constexpr (j + kA < NMC) ring[j % kA] = operand(std::integral_constant<int, j + kA>{}, lq, lg);
        else ring[j % kA] = operand(std::integral_constant<int, j + kA - NMC>{}, nq, ng);
        if constexpr (j < PK * DB) {
          dvt[j % DB] = O_::mfma(a, pp[j / DB], dvt[j % DB]);
        } else {
          constexpr int m = j - PK * DB;
          dkt[m % DB] = O_::mfma(a, dsp[m / DB], dkt[m % DB]);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // step u: copies of tile u + 2, then tile u - 1 (its Q/dO in buffer
    // (u - 1) % 4, its exchange block in buffer (u - 1) % 2)
    auto step_of = [&](auto active) __attribute__((always_inline)) {
      return [&, active](int u, auto par) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        using I = std::integral_constant<int, P>;
        using Im1 = std::integral_constant<int, P + 3>;
        using I2 = std::integral_constant<int, P + 2>;
        // vmcnt(0): this wave's copies of tile u + 1 are done. lgkmcnt(kA):
        // all but its last kA LDS reads are done; those are the ring reads of
        // tile u (LDS reads complete in order)
        static_assert(kA < 16, "lgkmcnt field");
        __builtin_amdgcn_s_waitcnt(0x0070 | (kA << 8));
        sync::bare_barrier();
        if (u + 2 < n_t) issue(t_begin + u + 2, bq(I2{}), bg(I2{}), bl(I2{}), bd(I2{}));
        if constexpr (decltype(active)::value) tile(bq(Im1{}), bg(Im1{}), bx(Im1{}), bq(I{}), bg(I{}));
        else prefetch(bq(I{}), bg(I{}));
      };
    };
    // prologue: tile 0 complete and visible, tile 1 in flight
    if (n_t > 0) issue(t_begin, lds_q0, lds_g0, lds_l0, lds_d0);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    if (n_t > 1) issue(t_begin + 1, lds_q1, lds_g1, lds_l1, lds_d1);
    sync::bare_barrier();
    // step u works on tile u - 1: idle for u <= f (no tile, or tiles the
    // pair skips), active after
    run4(0, min(f + 1, n_t + 1), step_of(std::integral_constant<bool, false>{}));
    run4(f + 1, n_t + 1, step_of(std::integral_constant<bool, true>{}));
    // dK = scale * dK^T, dV = dV^T (lane = key, registers = head-dim index),
    // stored as whole rows through one Q tile buffer per pair (free once
    // every wave has left the tile loop; no copy is in flight)
    __builtin_amdgcn_s_waitcnt(0x0070);
    sync::bare_barrier();
    const int nrows = min(kBKV, p.Nk - k0);
    const uint32_t range = (uint32_t)(nrows - 1) * row_bytes + 2 * D;
    const auto out_k = make_rsrc(p.dk + kvo + (size_t)k0 * rs, range);
    const auto out_v = make_rsrc(p.dv + kvo + (size_t)k0 * rs, range);
    uint8_t* const slot = pair == 0 ? lds_q0 : pair == 1 ? lds_q1 : pair == 2 ? lds_q2 : lds_q3;
    const uint32_t gbase = (uint32_t)(pair * 32) * row_bytes;
    store_rows<O_, D>(dkt, -p.scale, slot, out_k, gbase, row_bytes, lane);  // dkt holds -dK^T
    store_rows<O_, D>(dvt, 1.f, slot, out_v, gbase, row_bytes, lane);
  }
}

}  // namespace mha
