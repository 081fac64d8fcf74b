// Fused multi-head attention forward for gfx950 (CDNA4).
//
// One workgroup (8 wave64 waves) owns BQ = 256 query rows of one (batch,
// head), 32 per wave, and streams that head's keys and values through LDS in
// tiles of BK = 64 keys. Per key tile each wave, for its 32 query rows:
//
//   1. S^T = K_tile . Q^T on MFMA 32x32x16 (bf16/f16 in, fp32 accumulate);
//   2. masks scores only on tiles that cross the causal diagonal or the end
//      of the keys; tiles wholly past the causal frontier are never loaded;
//   3. online softmax: running row max m and row sum l, O rescaled by
//      alpha = exp(scale*(m_old - m_new)) when the max has grown (the
//      tile's row max itself is taken only when its P, computed against
//      the running max first, sum past the deferral bound below);
//   4. converts P to bf16/f16 in registers and accumulates O^T += V^T . P^T
//      on MFMA.
// After the last tile O is divided by l, rounded to the I/O type and written
// once; LSE = scale*m + ln(l) is written in fp32.
//
// Sources: the fused per-thread-block loop (read a Q block once, then for
// every K/V block compute S, the online softmax, the layout change of P and
// O += P V on chip, writing O in the last iteration) is "SparkAttention",
// Fig. 6 passage; sequence parallelism (several workers per head, each owning
// a block of query rows, no communication) is the FlashAttention
// long-sequence post, "Attention parallelism"; double-buffered K/V staging
// with the next tile's copy issued before the current tile's compute is the
// "CANN ops-transformer" article, sections 2.2 and 3.2; the running m and l
// and LSE = m + log l, and skipping whole tiles past the causal frontier, are
// "StreamKL", Methodology sections 1-2.
//
// gfx950 choices (not from the pages):
// * Ping-pong of two wave groups. Waves 0-3 and 4-7 each alternate a GEMM
//   phase (P.V of the previous tile and S^T of the current tile, 32 MFMAs;
//   a wave's first phase has no P.V, its last no S^T) and a softmax phase
//   (VALU), the second group half a period behind the
//   first: every SIMD holds one wave of each group, so one issues MFMAs
//   while the other runs its softmax. One workgroup barrier per key tile
//   (period) covers the reuse of the K and V buffers; within a period the
//   groups are not forced into step.
// * S is computed transposed (keys are MFMA rows, queries are columns), so
//   each lane owns one query: the row max needs one exchange between lanes
//   l and l^32, the row sum needs none until the end, and alpha is a
//   per-lane scalar for the O^T accumulator.
// * The rows of the K operand are fed in an order (bits 2 and 3 of the row
//   index swapped) that leaves every lane of the S^T accumulator holding 8
//   consecutive keys per 16-key step -- exactly the B-operand fragment of the
//   P.V product, so P needs no cross-lane layout change ("SparkAttention"
//   step 3 becomes a register-local conversion).
// * K and V tiles are copied global -> LDS by buffer loads that write LDS
//   directly (no staging registers); rows past the end of the keys read as
//   zero through the buffer's range check, so the tail needs no branches.
//   The V^T operand of the P.V product comes from two LDS transpose reads
//   (ds_read_b64_tr_b16) of the row-major V tile per MFMA.
// * The row max is exchanged between the two lane halves with
//   v_permlane32_swap; barriers are bare s_barrier instructions with the
//   needed waits made explicit.
// * LDS tiles are XOR-swizzled in 16-byte units so the MFMA operand reads
//   (row reads of K, transpose reads of V) are free of bank conflicts; the
//   GEMM phase reads each operand three MFMAs ahead of its use.
// * The O rescale is deferred while a row's max stays within 2^8 (exp2
//   domain) of the max O and l were last scaled to; O/l and LSE are the same
//   in exact arithmetic, and the rescale then runs only when the max jumps.
//   Since every P is at most its lane's tile sum, a tile whose sums stay
//   within 2^8 needs no row max at all; element masks are one compare of
//   a constant offset with a per-lane limit.
// * The 1-D grid is remapped so that all query tiles of a head run on one
//   XCD (workgroups are dispatched round-robin over the 8 XCDs), keeping the
//   head's K/V in that XCD's L2; heads are taken in groups small enough for
//   their K/V to stay in L2 while in flight; each XCD starts its heaviest
//   causal query tiles first, ordered for its four shader engines.
// * The epilogue stages each wave's O rows in LDS and writes whole rows
//   with 16-byte stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mha_tiles.hpp"

namespace mha {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct BF16 {};
struct F16 {};

template <typename T>
struct Ops;

template <>
struct Ops<BF16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Two fp32 -> packed 2 x bf16, round to nearest even.
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  // Row-sum update for two probabilities: in fp32 (bf16 keeps 8 significant
  // bits, too few for the LSE bound on rows with few keys).
  static __device__ __forceinline__ float sum2(uint32_t, float x, float y, float acc) {
    return acc + x + y;
  }
};

template <>
struct Ops<F16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // Two fp32 -> packed 2 x f16, round to nearest even.
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  // Row-sum update for two probabilities from their packed f16 values: one
  // v_dot2 with (1, 1) (f16 keeps 11 significant bits).
  static __device__ __forceinline__ float sum2(uint32_t packed, float, float, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), one, acc, false);
  }
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, H, Nq, Nk;
  float scale;       // softmax scale (> 0)
  float scale_log2;  // scale * log2(e): exp(scale*x) = exp2(scale_log2*x)
  float defer_raw;   // rescale threshold in raw-score units: 8 / scale_log2
  int n_qtiles;      // ceil(Nq / BQ)
  int n_blocks;      // B * H * n_qtiles
};

// kWaves (two groups of four: one wave of each per SIMD), kThreads, kBQ
// (query rows per workgroup, 32 per wave) and kBK (keys per tile) are in
// mha_tiles.hpp.
// The O rescale is deferred while a row's running max stays within 2^8 (in
// the exp2 domain) of the reference max the accumulators were scaled to.
constexpr float kDeferLog2 = 8.0f;
constexpr float kDeferSum = 256.0f;  // 2^kDeferLog2

// Row index of the K operand fed to MFMA row m: bits 2 and 3 of m swapped
// (an involution).
__device__ __forceinline__ int k_row_order(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// 16-byte-chunk swizzles of the K and V rows in LDS. They are chosen so that
// the lanes of one LDS pass hit distinct banks whether the LDS serves 8 lanes
// x 16 bytes (b128) / 16 lanes x 8 bytes (b64) per 128-byte pass, or 16 x 16
// / 32 x 8 per 256-byte pass.
//  K, read as S^T A-operand rows: lane m (of 16) reads row k_row_order(m).
template <int D>
__device__ __forceinline__ int k_swz(int key) {
  const int m = k_row_order(key & 15);
  if constexpr (D == 128) return m;            // 16 chunks per 256-byte row
  else return (m >> 1) ^ (4 * (m & 1));        // 8 chunks per 128-byte row
}
// Workgroup order within one XCD. The XCD hands its k-th workgroup to
// shader engine k mod 4 (8 CUs each) strictly in order: a workgroup waits
// for a free CU in its own engine and the ones behind it wait too. With
// work ranked heaviest first and S workgroups resident on the XCD at a time,
// reversing each group of four in every even round of S puts the lightest
// of each group on engine 0 there, so engines free their CUs in the order
// the next workgroups are bound for them and heavy and light work pair up
// on every CU (a simulation of this dispatch reaches the ideal per-CU load
// on the causal grids). Returns the rank workgroup k takes among n.
__device__ __forceinline__ int engine_order(int k, int n, int S) {
  return (((k / S) & 1) == 0 && (k | 3) < n) ? (k ^ 3) : k;
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// max / sum of x over lanes l and l ^ 32, in both lanes: one v_permlane32_swap
// (a VALU op) instead of a shuffle through LDS. With both operands x, the
// swap returns x of lanes 0-31 in every lane (first result) and x of lanes
// 32-63 in every lane (second result). The results are read as plain
// integers first: __builtin_bit_cast of a vector element reads element 0.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  const uint32_t lo = r[0], hi = r[1];
  return fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  const uint32_t lo = r[0], hi = r[1];
  return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// One wave copies 1 KiB global -> LDS: lane l's 16 bytes at `voffset` land at
// lds_dst + 16*l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)((lds_u8*)lds_dst),
                                           16, voffset, 0, 0, 0);
}

// The same copy issued by inline asm: the compiler then does not treat it as
// an LDS write and adds no wait for it before later LDS reads (it cannot
// tell the buffer being filled from the ones being read, so it would wait
// for every copy in flight). Code that uses it waits explicitly (vmcnt) and
// passes a barrier before reading what it copied.
__device__ __forceinline__ void dma16_async(__amdgpu_buffer_rsrc_t r, uint8_t* lds_dst, uint32_t voffset) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8*)lds_dst);
  // M0 holds the LDS address; s_nop: the copy may not read M0 in the cycle
  // after it was written
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(r), "{m0}"(m0)
               : "memory");
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS transpose read of 4 x 16-bit values: within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte pieces addressed by lanes i/4,
// 4 + i/4, 8 + i/4 and 12 + i/4.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* ptr) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)ptr));
  return __builtin_bit_cast(u32x2, r);
}

// 16-byte-chunk swizzle of the tiles that are read both as MFMA rows (16
// lanes read the 16 rows k_row_order(0..15) at one chunk) and by transpose
// reads (16 lanes read 4 consecutive rows x 2 chunks, 32 lanes 4 rows x 4
// chunks). With t = row & 3 and m = (row >> 2) & 3, the 16 rows of a row
// read get 16 (d = 128) or, per row parity, 8 (d = 64) different chunk
// positions, and the 4 rows of a transpose read put their chunks on
// disjoint positions, whether the LDS serves 128 or 256 bytes per pass.
// (The K tile's swizzle of the forward, made for row reads only, would give
// 4-way conflicts on the transpose reads.)
template <int D>
__device__ __forceinline__ int t_swz(int row) {
  const int t = row & 3, m = (row >> 2) & 3;
  const int gray = m ^ (m >> 1);
  if constexpr (D == 128) return (4 * t + 2 * (t >> 1)) ^ gray;  // 16 chunks per row
  else return (2 * t) ^ gray;                                    // 8 chunks per row
}

// Per-lane byte offsets of the transpose reads that form the A operand
// "rows = head-dim index 32*db + (lane % 32), k-slots = 8 consecutive tile
// rows 16*ks + 8*(lane / 32) + 0..7" from a row-major tile whose 16-byte
// chunks are swizzled by t_swz<D> of the row: two reads per operand, the
// second 4 rows further (r = 0, 1). Lane (g, a) of 16-lane group g supplies
// the 8-byte piece of row 8*(g/2) + 4r + a/4 at head-dim index
// 32*db + 16*(g%2) + 4*(a%4). Everything but these offsets (the 16-row step
// ks) is an immediate, since the swizzle depends on the row's low 4 bits.
template <int D>
__device__ __forceinline__ uint32_t tr_off(int lane, int db, int r) {
  constexpr int ROWB = 2 * D;
  const int g = lane >> 4, a = lane & 15;
  const int row = 8 * (g >> 1) + 4 * r + (a >> 2);
  const int chunk = 4 * db + 2 * (g & 1) + ((a & 3) >> 1);
  return row * ROWB + 16 * (chunk ^ t_swz<D>(row)) + 8 * (a & 1);
}

// The 8 values of one transposed A operand.
__device__ __forceinline__ u32x4 tr_operand(const uint8_t* base, uint32_t off0, uint32_t off1) {
  const u32x2 t0 = lds_read_tr16(base + off0);
  const u32x2 t1 = lds_read_tr16(base + off1);
  return u32x4{t0[0], t0[1], t1[0], t1[1]};
}

// One wave's 32 output rows, held in MFMA-accumulator layout (lane (ln, hf)
// owns row ln; value r of block db is column 32db + 8(r/4) + 4hf + r%4),
// scaled by `mul`, rounded to the I/O type and written out through an LDS
// slot of 32 * 2D bytes: each lane's eight-byte pieces, scattered over its
// row, are staged (row ln, 16-byte chunk c at chunk c ^ (ln mod D/8), which
// spreads the writes over the banks) and leave as 16-byte buffer stores
// that cover whole rows. `gbase` is the byte offset of the wave's first row
// in the buffer `out`; rows past its range are dropped by the range check.
template <typename Ops_, int D>
__device__ __forceinline__ void store_rows(const f32x16* acc, float mul, uint8_t* slot,
                                           __amdgpu_buffer_rsrc_t out, uint32_t gbase,
                                           uint32_t row_bytes, int lane) {
  constexpr int DB = D / 32, CH = D / 8, ROWB = 2 * D, RPC = 1024 / ROWB, NC = 32 * ROWB / 1024;
  const int ln = lane & 31, hf = lane >> 5;
  const uint32_t y = (uint32_t)(ln & (CH - 1)), wa = (uint32_t)(ln * ROWB + 8 * hf);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      u32x2 w2;
      w2[0] = Ops_::pack(acc[db][4 * a + 0] * mul, acc[db][4 * a + 1] * mul);
      w2[1] = Ops_::pack(acc[db][4 * a + 2] * mul, acc[db][4 * a + 3] * mul);
      *reinterpret_cast<u32x2*>(slot + wa + 16 * (y ^ (uint32_t)(4 * db + a))) = w2;
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slot is written
  // copy c reads slot rows c*RPC + lane/CH at physical chunk lane % CH
  const uint32_t rl = (uint32_t)lane / CH, pc = (uint32_t)lane % CH;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(slot + c * 1024 + 16 * lane);
    const uint32_t lc = (pc ^ ((uint32_t)(c * RPC) + rl)) & (CH - 1);  // logical chunk
    __builtin_amdgcn_raw_buffer_store_b128(w, out, gbase + ((uint32_t)(c * RPC) + rl) * row_bytes + 16 * lc, 0, 0);
  }
}

// Scheduling pins for a GEMM phase that runs MFMAs N .. NE-1 (the first NPV
// take two operand reads, the rest one): the reads of the first AHEAD
// operands, then for every MFMA n one MFMA followed by the reads of operand
// n+AHEAD.
template <int N, int NPV, int NE, int AHEAD>
struct PinInterleave {
  static constexpr int reads_of(int n) { return n < NPV ? 2 : 1; }
  // the reads before MFMA N (the phase's first)
  static constexpr int preload() {
    int r = 0;
    for (int n = N; n < N + AHEAD && n < NE; ++n) r += reads_of(n);
    return r;
  }
  static __device__ __forceinline__ void pin_preload() {
    __builtin_amdgcn_sched_group_barrier(0x100, preload(), 0);
  }
  static __device__ __forceinline__ void apply() {
    if constexpr (N < NE) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (N + AHEAD < NE)
        __builtin_amdgcn_sched_group_barrier(0x100, reads_of(N + AHEAD), 0);
      PinInterleave<N + 1, NPV, NE, AHEAD>::apply();
    }
  }
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void mha_fwd_kernel(Params p) {
  using O_ = Ops<T>;
  constexpr int BK = kBK;
  constexpr int KB = BK / 32;            // 32-key blocks per tile (S^T row blocks)
  constexpr int DK = D / 16;             // k-steps of Q.K^T over the head dim
  constexpr int DB = D / 32;             // 32-row blocks of O^T
  constexpr int PK = BK / 16;            // k-steps of P.V over the keys
  constexpr int CH = D / 8;              // 16-byte chunks per K/V row
  constexpr int ROWB = D * 2;            // bytes per K/V row in LDS
  constexpr int TILEB = BK * ROWB;       // bytes per K or V tile
  constexpr int RPI = 1024 / ROWB;       // rows per 1 KiB wave copy
  constexpr int NCPW = TILEB / 1024 / kWaves;  // 1 KiB copies per wave per tensor
  static_assert(NCPW >= 1, "tile too small for the workgroup");

  constexpr int OSB = 32 * ROWB;  // one wave's 32 output rows
  // One LDS allocation laid out by hand: the K and V tiles first, so the
  // GEMM phases address them with immediate offsets (below 64 KiB), then one
  // output-staging slot per wave for the epilogue.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * TILEB + 2 * TILEB + kWaves * OSB];
  uint8_t* const lds_k0 = lds;
  uint8_t* const lds_k1 = lds + TILEB;
  uint8_t* const lds_v0 = lds + 2 * TILEB;  // V tiles: row-major, chunks swizzled by t_swz
  uint8_t* const lds_v1 = lds + 2 * TILEB + TILEB;
  uint8_t* const lds_o = lds + 2 * TILEB + 2 * TILEB;

  // ---- work item: (batch, head, query tile) --------------------------------
  // Workgroups are dispatched in index order, round-robin over the 8 XCDs.
  // When the heads split evenly over the XCDs, XCD x takes the heads
  // bh = 8*i + x (a head's K/V then stays in one XCD's L2) and its k-th
  // workgroup takes query-tile rank k / (heads per XCD) of head rank
  // k % (heads per XCD); otherwise the same order runs over all heads. For
  // causal attention query-tile rank 0 is the last (heaviest) query tile, so
  // every XCD starts its heaviest work first.
  const int lin = blockIdx.x;
  const int BH = p.B * p.H;
  const bool by_xcd = (BH & 7) == 0;
  int k = by_xcd ? lin >> 3 : lin;
  const int nh = by_xcd ? BH >> 3 : BH;
  if (by_xcd) k = engine_order(k, nh * p.n_qtiles, 32);  // one workgroup per CU
  // Heads are taken in groups of G, enough for the query tiles of one group
  // to fill the XCD's 32 CUs (or all 256): the workgroups running at one
  // time then stream the K/V of only G heads, which stay in L2.
  const int G = min(nh, max(1, ((by_xcd ? 32 : 256) + p.n_qtiles - 1) / p.n_qtiles));
  const int g = k / (G * p.n_qtiles);
  const int gr = k - g * (G * p.n_qtiles);
  const int gn = min(G, nh - g * G);  // heads in this group (the last may be short)
  const int qi = gr / gn;
  const int hh = g * G + (gr - qi * gn);
  const int bh = by_xcd ? 8 * hh + (lin & 7) : hh;
  const int qt = CAUSAL ? p.n_qtiles - 1 - qi : qi;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int q0 = qt * kBQ;

  const size_t rs = (size_t)p.H * D;  // elements between consecutive tokens
  const uint16_t* __restrict__ Qb = p.q + ((size_t)b * p.Nq * p.H + h) * D;
  const uint16_t* __restrict__ Kb = p.k + ((size_t)b * p.Nk * p.H + h) * D;
  const uint16_t* __restrict__ Vb = p.v + ((size_t)b * p.Nk * p.H + h) * D;
  uint16_t* __restrict__ Ob = p.o + ((size_t)b * p.Nq * p.H + h) * D;
  const uint32_t row_bytes = (uint32_t)(rs * 2);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;       // 0: group A, 1: group B (half a period later)
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int qw0 = q0 + wave * 32;  // first query row of this wave
  const int my_q = qw0 + ln;       // query row owned by this lane

  // ---- Q fragments (B operand of S^T), read once ---------------------------
  // The wave's 32 Q rows are copied whole (1 KiB per copy) into its
  // output-staging slot, which the epilogue only needs later; row r's
  // 16-byte chunk c lands at chunk c ^ (r mod CH) so the fragment reads
  // spread over the banks. Rows past Nq read as zero.
  u32x4 qf[DK];
  {
    constexpr int RPC = 1024 / ROWB;  // rows per copy
    const int nrows = min(kBQ, p.Nq - q0);
    const auto r = make_rsrc(Qb + (size_t)q0 * rs, (uint32_t)(nrows - 1) * row_bytes + ROWB);
    const uint32_t rl = (uint32_t)lane / CH, pc = (uint32_t)lane % CH;
#pragma unroll
    for (int c = 0; c < OSB / 1024; ++c) {
      const uint32_t row = (uint32_t)(c * RPC) + rl;  // row within the wave's 32
      dma16(r, lds_o + wave * OSB + c * 1024,
            (uint32_t)(wave * 32 + row) * row_bytes + 16 * ((pc ^ row) & (CH - 1)));
    }
  }
  auto read_q = [&]() __attribute__((always_inline)) {
    const uint8_t* qs = lds_o + wave * OSB + ln * ROWB;
#pragma unroll
    for (int i = 0; i < DK; ++i)
      qf[i] = *reinterpret_cast<const u32x4*>(qs + 16 * ((2 * i + hf) ^ (ln & (CH - 1))));
  };

  // ---- key tiles this query tile needs -------------------------------------
  const int n_ktiles_all = (p.Nk + BK - 1) / BK;
  int n_kt = n_ktiles_all;
  if (CAUSAL) {
    const int qmax = min(p.Nq, q0 + kBQ);  // one past the last visible query
    n_kt = min(n_ktiles_all, (qmax + BK - 1) / BK);
  }
  // Tiles [0, jm) need no element mask for this wave's rows; later ones may
  // (the last, partial tile; tiles reaching past row qw0 when causal).
  int jm = (p.Nk % BK) ? p.Nk / BK : n_ktiles_all;
  if (CAUSAL) jm = min(jm, (qw0 + 1) / BK);
  // Tiles from j_end on lie wholly past this wave's rows (causal) or past
  // the keys: this wave skips them.
  const int j_end = CAUSAL ? min(n_kt, qw0 / BK + 1) : n_kt;

  // ---- asynchronous global -> LDS copies ------------------------------------
  uint32_t k_off[NCPW];
#pragma unroll
  for (int it = 0; it < NCPW; ++it) {
    const int row = (it * kWaves + wave) * RPI + lane / CH;
    const int pc = lane % CH;  // physical chunk in LDS
    k_off[it] = row * row_bytes + 16 * (pc ^ k_swz<D>(row));
  }
  // A tile j >= n_kt gets an empty range: its copies read nothing.
  auto rsrc_for = [&](const uint16_t* base, int j) __attribute__((always_inline)) {
    const int kbase = j * BK;
    const int nvalid = min(BK, p.Nk - kbase);
    return make_rsrc(base + (size_t)kbase * rs, j < n_kt ? (uint32_t)(nvalid - 1) * row_bytes + ROWB : 0u);
  };
  auto issue_k = [&](int j, uint8_t* lk) __attribute__((always_inline)) {
    const auto r = rsrc_for(Kb, j);
#pragma unroll
    for (int it = 0; it < NCPW; ++it) dma16_async(r, lk + (it * kWaves + wave) * 1024, k_off[it]);
  };
  // V tiles are copied like K, row-major, 16-byte chunks swizzled by
  // t_swz<D> of the row so the transpose reads of the P.V operand are
  // conflict-free.
  uint32_t v_off[NCPW];
#pragma unroll
  for (int it = 0; it < NCPW; ++it) {
    const int row = (it * kWaves + wave) * RPI + lane / CH;
    v_off[it] = row * row_bytes + 16 * ((lane % CH) ^ t_swz<D>(row));
  }
  auto issue_v = [&](int j, uint8_t* lv) __attribute__((always_inline)) {
    const auto r = rsrc_for(Vb, j);
#pragma unroll
    for (int it = 0; it < NCPW; ++it) dma16_async(r, lv + (it * kWaves + wave) * 1024, v_off[it]);
  };

  // ---- per-lane LDS read offsets (fixed for the whole kernel) ---------------
  // K operand: MFMA row ln reads key kb*32 + k_row_order(ln); its chunk
  // swizzle depends only on the key's low 4 bits, i.e. only on ln, so one
  // offset per k-step serves both 32-key blocks (+32 rows) and both buffers.
  uint32_t koff[DK];
  {
    const int key = k_row_order(ln);
    const int sw = k_swz<D>(key);
#pragma unroll
    for (int i = 0; i < DK; ++i) koff[i] = key * ROWB + 16 * ((2 * i + hf) ^ sw);
  }
  // V^T operand: two transpose reads of the row-major V tile per MFMA
  uint32_t toff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 2; ++r) toff[db][r] = tr_off<D>(lane, db, r);

  // ---- running state -------------------------------------------------------
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  f32x16 s[KB];             // S^T of the tile between its GEMM and softmax phases
  u32x4 pf[PK];             // packed P^T between the softmax and the next GEMM phase
#pragma unroll
  for (int ks = 0; ks < PK; ++ks) pf[ks] = u32x4{0, 0, 0, 0};
  float m_run = -INFINITY;  // reference max (raw scores q.k) of o and l_run
  float l_run = 0.f;        // this lane's part of the row sum
  const float c = p.scale_log2;

  // GEMM phase of tile j: O^T += V_{j-1}^T P_{j-1}^T, then S^T_j = K_j Q^T.
  // The 16 + 16 MFMAs are one straight-line sequence; the LDS operand of
  // MFMA n+kAhead is read while MFMA n issues, so LDS latency stays hidden
  // behind MFMA work. The per-lane offsets pass through an empty asm so the
  // compiler forms each address here (buffer base in the instruction's
  // immediate offset) instead of hoisting one register per (buffer, step).
  constexpr int NPV = PK * DB;  // P.V MFMAs per tile
  constexpr int NS = DK * KB;   // S^T MFMAs per tile
  constexpr int kAhead = 3;
  // The phase of tile 0 has no P.V part and a wave's phase j = j_end, after
  // its last tile, no S^T part (KIND 1 and 2, compile time); the middle
  // phases share one code path, so O stays in the same registers throughout.
  // `copies` issues this wave's tile copies right after the first operand
  // reads (their latency hides the issue) and before the first MFMA.
  auto gemm = [&](int j, const uint8_t* lk, const uint8_t* lv, auto copies, auto kind)
                  __attribute__((always_inline)) {
    constexpr int N0 = decltype(kind)::value == 1 ? NPV : 0;         // first MFMA
    constexpr int NE = decltype(kind)::value == 2 ? NPV : NPV + NS;  // one past the last
    uint32_t ko[DK];
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      ko[i] = koff[i];
      asm volatile("" : "+v"(ko[i]));
    }
    // operand of MFMA n: n < NPV -> V^T fragment (ks, db) = (n / DB, n % DB);
    // else K fragment (i, kb) = ((n - NPV) / KB, (n - NPV) % KB)
    auto load_op = [&](int n) __attribute__((always_inline)) -> u32x4 {
      u32x4 a;
      if (n < NPV) {
        const int ks = n / DB, db = n % DB;
        a = tr_operand(lv + ks * 16 * ROWB, toff[db][0], toff[db][1]);
      } else {
        const int m = n - NPV, i = m / KB, kb = m % KB;
        a = *reinterpret_cast<const u32x4*>(lk + ko[i] + kb * 32 * ROWB);
      }
      return a;
    };
    // the first operand reads, then the copies
    u32x4 buf[kAhead];
#pragma unroll
    for (int n = N0; n < N0 + kAhead && n < NE; ++n) buf[n % kAhead] = load_op(n);
    copies();
    PinInterleave<N0, NPV, NE, kAhead>::pin_preload();
    if (j > j_end) return;  // guard (wave-uniform): the loops stop at j_end
    if constexpr (NE > NPV) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    }
#pragma unroll
    for (int n = N0; n < NE; ++n) {
      const u32x4 a = buf[n % kAhead];
      if (n + kAhead < NE) buf[n % kAhead] = load_op(n + kAhead);
      if (n < NPV) {
        const int ks = n / DB, db = n % DB;
        o[db] = O_::mfma(a, pf[ks], o[db]);
      } else {
        const int m = n - NPV, i = m / KB, kb = m % KB;
        s[kb] = O_::mfma(a, qf[i], s[kb]);
      }
    }
    // pin the order: per MFMA the reads kAhead ahead
    PinInterleave<N0, NPV, NE, kAhead>::apply();
  };

  // Softmax phase of tile j: mask, running max, exp, row sum, P^T fragments.
  auto softmax = [&](int j) __attribute__((always_inline)) {
    if (j >= j_end) return;  // guard: the loops call it for j < j_end only
    const int k0 = j * BK;
    if (j >= jm) {
      // the empty asm keeps the compiler from turning this rarely taken,
      // wave-uniform branch into selects executed on every tile
      asm volatile("" ::: "memory");
      // element (kb, r) is key k0 + 8*hf + off with off = 32*kb + 16*(r>>3)
      // + (r&7); it is visible iff key < Nk and (causal) key <= my_q, i.e.
      // iff off <= lim: one compare with a constant per element
      const int lim = (CAUSAL ? min(p.Nk - 1, my_q) : p.Nk - 1) - k0 - 8 * hf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + 16 * (r >> 3) + (r & 7);
          s[kb][r] = off <= lim ? s[kb][r] : -INFINITY;
        }
    }
    // The exact step: row max of the tile (two independent chains, one per
    // 32-key block, then across halves); the O and l rescale is deferred
    // while the max stays within kDeferLog2 of the reference max m_run.
    auto max_and_rescale = [&]() __attribute__((always_inline)) {
      float mk[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        mk[kb] = s[kb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mk[kb] = fmaxf(mk[kb], s[kb][r]);
      }
      float mx = mk[0];
#pragma unroll
      for (int kb = 1; kb < KB; ++kb) mx = fmaxf(mx, mk[kb]);
      mx = max_halves(mx);
      if (__any(mx > m_run + p.defer_raw)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2((m_run - m_new) * c);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m_run = m_new;
      }
    };
    // P = exp(scale*(s - m_run)) into the P^T fragments (k-step ks covers
    // keys 16*ks + 8*hf + 0..7), leaving s as it is; returns the lane's
    // part of the tile's row sum (PK independent chains)
    auto exp_pack = [&]() __attribute__((always_inline)) -> float {
      const float mc = m_run * c;
      float rsum[PK];
#pragma unroll
      for (int ks = 0; ks < PK; ++ks) {
        const int kb = ks >> 1, r0 = 8 * (ks & 1);
        // (chains from 0: seeding them with the first pair saves an add
        // but changes the compiler's order of the exponentials, packs and
        // adds, which measured 2 % slower at d = 128)
        rsum[ks] = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float x0 = fast_exp2(__builtin_fmaf(s[kb][r0 + 2 * t], c, -mc));
          const float x1 = fast_exp2(__builtin_fmaf(s[kb][r0 + 2 * t + 1], c, -mc));
          pf[ks][t] = O_::pack(x0, x1);
          rsum[ks] = O_::sum2(pf[ks][t], x0, x1, rsum[ks]);
        }
      }
#pragma unroll
      for (int ks = 1; ks < PK; ++ks) rsum[0] += rsum[ks];
      return rsum[0];
    };
    // The row max only decides whether the reference max moves, i.e.
    // whether some score exceeds m_run by more than the deferral bound.
    // Every P is at most the lane's tile sum, so a sum within 2^kDeferLog2
    // on every lane shows that no score crossed the bound, and the max is
    // not needed: the P taken against m_run are those the exact step gives.
    // Otherwise (and on the first tile, before m_run is set) the exact
    // step runs and P is taken again. The test is written so that a NaN
    // or infinite sum (scores far past m_run) fails it.
    bool exact = j == 0;
    float rt = 0.f;
    if (!exact) {
      rt = exp_pack();
      exact = __any(!(rt <= kDeferSum));
    }
    if (exact) {
      max_and_rescale();
      rt = exp_pack();
    }
    l_run += rt;
  };

  // ---- period schedule -----------------------------------------------------
  // Key tile j takes period j, between barrier #j (#0 ends the prologue)
  // and barrier #j+1. Group A (grp 0) runs the GEMM phase of tile j and then
  // its softmax in period j; group B runs the softmax of tile j-1 and then
  // the GEMM phase of tile j, so on every SIMD one wave issues MFMAs while
  // the other runs its softmax. Each group has its own straight-line loop;
  // the k-th barrier of every wave pairs up. K_j is read in period j, V_j
  // in period j+1.
  // * Early in period m every wave starts its share of the LDS copies of
  //   K_{m+1}, into the K buffer that held K_{m-1}, and of V_m, into the V
  //   buffer that held V_{m-2} (both last read in period m-1): group B right
  //   after barrier #m, group A inside its GEMM phase, after its first
  //   operand reads. They are waited for before barrier #m+1.
  // Workgroup barrier without a memory fence: __syncthreads() also releases
  // memory at workgroup scope, which would make each wave wait at every
  // barrier for the K copy it started at the beginning of the period. The
  // waits that matter are explicit (wait_k: the copies the next period reads
  // and this wave's LDS writes); the empty asm statements keep the compiler
  // from moving LDS accesses across the barrier.
  auto barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // K_{m+1} and V_m landed.
  auto wait_k = [&](bool) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
  };
  // K_{m+1} copy into K buffer (m+1) & 1 and V_m copy into V buffer m & 1;
  // BUF = m & 1 (compile time).
  auto issue_k_next = [&](int m, auto buf) __attribute__((always_inline)) {
    if constexpr (decltype(buf)::value == 0) {
      if (m + 1 < n_kt) issue_k(m + 1, lds_k1);
      if (m < n_kt) issue_v(m, lds_v0);
    } else {
      if (m + 1 < n_kt) issue_k(m + 1, lds_k0);
      if (m < n_kt) issue_v(m, lds_v1);
    }
  };
  // The same for m < n_kt without a branch, so that it can sit inside a GEMM
  // phase: for m + 1 = n_kt the K copy has an empty range and reads nothing.
  auto issue_k_next_inline = [&](int m, auto buf) __attribute__((always_inline)) {
    if constexpr (decltype(buf)::value == 0) {
      issue_k(m + 1, lds_k1);
      issue_v(m, lds_v0);
    } else {
      issue_k(m + 1, lds_k0);
      issue_v(m, lds_v1);
    }
  };
  auto no_copies = []() __attribute__((always_inline)) {};
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // GEMM phase of tile j with BUF = j & 1: K_j in K buffer BUF, V_{j-1} in
  // V buffer BUF ^ 1; KIND as for gemm (default: a middle phase).
  auto gemm_phase = [&](int j, auto buf, auto copies, auto kind) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(2);
    if constexpr (decltype(buf)::value == 0)
      gemm(j, lds_k0, lds_v1, copies, kind);
    else
      gemm(j, lds_k1, lds_v0, copies, kind);
    __builtin_amdgcn_s_setprio(0);
  };

  issue_k(0, lds_k0);
  wait_k(true);  // Q and K_0 landed
  read_q();
  barrier();     // #0
  if (grp == 0) {
    // group A: period j = GEMM(j), softmax(j)
    auto tile = [&](int j, auto buf, auto kind) __attribute__((always_inline)) {
      // start of period j: the copies go out inside the GEMM phase
      gemm_phase(j, buf, [&]() __attribute__((always_inline)) { issue_k_next_inline(j, buf); }, kind);
      softmax(j);
      wait_k(j + 1 < n_kt);
      barrier();                // end of period j
    };
    tile(0, I0{}, I1{});
    int j = 1;
    for (; j + 1 < j_end; j += 2) {
      tile(j, I1{}, I0{});
      tile(j + 1, I0{}, I0{});
    }
    if (j < j_end) {
      tile(j, I1{}, I0{});
      ++j;
    }
    // period j_end: P.V of the wave's last tile; for j_end < n_kt (causal,
    // rows above the workgroup's last) the wave then only copies its share
    // of the tiles and meets the barriers until the workgroup is done
    if (j < n_kt) {
      if (j & 1) issue_k_next(j, I1{});
      else issue_k_next(j, I0{});
    }
    if (j & 1) gemm_phase(j, I1{}, no_copies, I2{});
    else gemm_phase(j, I0{}, no_copies, I2{});
    for (; j < n_kt; ++j) {
      if (j > j_end) {
        if (j & 1) issue_k_next(j, I1{});
        else issue_k_next(j, I0{});
      }
      wait_k(true);
      barrier();                // end of period j
    }
  } else {
    // group B: period j = softmax(j-1), GEMM(j)
    issue_k_next(0, I0{});      // start of period 0
    auto tile = [&](int j, auto buf, auto kind) __attribute__((always_inline)) {
      gemm_phase(j, buf, no_copies, kind);
      wait_k(j + 1 < n_kt);
      barrier();                // end of period j
      if constexpr (decltype(buf)::value == 0)
        issue_k_next(j + 1, I1{});  // start of period j+1
      else
        issue_k_next(j + 1, I0{});
      softmax(j);
    };
    tile(0, I0{}, I1{});
    int j = 1;
    for (; j + 1 < j_end; j += 2) {
      tile(j, I1{}, I0{});
      tile(j + 1, I0{}, I0{});
    }
    if (j < j_end) {
      tile(j, I1{}, I0{});
      ++j;
    }
    // period j_end: P.V of the wave's last tile, then (j_end < n_kt) copies
    // and barriers only
    if (j & 1) gemm_phase(j, I1{}, no_copies, I2{});
    else gemm_phase(j, I0{}, no_copies, I2{});
    for (; j < n_kt; ++j) {
      wait_k(true);
      barrier();                // end of period j
      if (j & 1) issue_k_next(j + 1, I0{});  // start of period j+1
      else issue_k_next(j + 1, I1{});
    }
  }

  // ---- epilogue: O = O^T / l, LSE = scale*m + ln(l) ------------------------
  // Each lane holds one query row's O as 8-byte pieces spread over the row;
  // written out directly they would be 16 scattered partial-line writes per
  // lane. They go through the wave's LDS slot instead (row ln, 16-byte
  // chunk c at c ^ (ln mod CH) so the writes spread over the banks) and
  // leave as 16-byte stores that cover whole rows. The buffer's range check
  // drops rows past Nq.
  const float l_tot = sum_halves(l_run);
  const float inv = 1.f / l_tot;
  {
    const int nrows = min(kBQ, p.Nq - q0);
    const auto o_rs = make_rsrc(Ob + (size_t)q0 * rs, (uint32_t)(nrows - 1) * row_bytes + ROWB);
    store_rows<O_, D>(o, inv, lds_o + wave * OSB, o_rs, (uint32_t)(wave * 32) * row_bytes, row_bytes, lane);
  }
  if (my_q < p.Nq && hf == 0) {
    const float lse = m_run * p.scale + fast_log2(l_tot) * 0.69314718055994531f;
    p.lse[((size_t)b * p.H + h) * p.Nq + my_q] = lse;
  }
}

}  // namespace mha
