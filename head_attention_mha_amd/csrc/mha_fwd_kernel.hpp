// Fused multi-head attention forward for gfx950 (CDNA4).
//
// One workgroup (4 wave64 waves) owns BQ = 128 query rows of one (batch, head)
// and streams that head's keys and values through LDS in tiles of BK = 64
// keys, double-buffered. Per key tile each wave, for its 32 query rows:
//
//   1. S^T = K_tile . Q^T on MFMA 32x32x16 (bf16/f16 in, fp32 accumulate);
//   2. masks scores only on tiles that cross the causal diagonal or the end
//      of the keys; tiles wholly past the causal frontier are never loaded;
//   3. online softmax: running row max m and row sum l, O rescaled by
//      alpha = exp(scale*(m_old - m_new));
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
// * S is computed transposed (keys are MFMA rows, queries are columns), so
//   each lane owns one query: the row max needs one exchange between lanes
//   l and l^32, the row sum needs none until the end, and alpha is a
//   per-lane scalar for the O^T accumulator.
// * The rows of the K operand are fed in an order (bits 2 and 3 of the row
//   index swapped) that leaves every lane of the S^T accumulator holding 8
//   consecutive keys per 16-key step -- exactly the B-operand fragment of the
//   P.V product, so P needs no cross-lane layout change ("SparkAttention"
//   step 3 becomes a register-local conversion).
// * V is transposed on its way into LDS: each thread loads two keys' 8-wide
//   rows and writes 32-bit words holding (V[2k][d], V[2k+1][d]); the V^T
//   operand is then one 16-byte LDS read per MFMA.
// * LDS tiles are XOR-swizzled in 16-byte units so the stores of the global
//   rows and the MFMA operand reads are free of bank conflicts.
// * The 1-D grid is remapped so that consecutive work items of one head land
//   on the same XCD (workgroups are dispatched round-robin over the 8 XCDs),
//   keeping a head's K/V in that XCD's L2; causal query tiles run heaviest
//   first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
  int n_qtiles;      // ceil(Nq / BQ)
  int n_blocks;      // B * H * n_qtiles
};

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;  // query rows per workgroup
constexpr int kBK = 64;           // keys per tile

// Row index of the K operand fed to MFMA row m: bits 2 and 3 of m swapped.
__device__ __forceinline__ int k_row_order(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// 16-byte-chunk swizzle of a K row in LDS (keeps 8 lanes of an operand read
// on distinct banks for the row order above).
__device__ __forceinline__ int k_swz(int key) { return (key & 3) | ((key >> 1) & 4); }
// 16-byte-group swizzle of a V^T row (row = head-dim index) in LDS.
__device__ __forceinline__ int vt_swz(int d) { return (d + (d >> 3)) & 7; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void mha_fwd_kernel(Params p) {
  using O_ = Ops<T>;
  constexpr int BK = kBK;
  constexpr int KB = BK / 32;       // 32-key blocks per tile (S^T row blocks)
  constexpr int DK = D / 16;        // k-steps of Q.K^T over the head dim
  constexpr int DB = D / 32;        // 32-row blocks of O^T
  constexpr int PK = BK / 16;       // k-steps of P.V over the keys
  constexpr int CH = D / 8;         // 16-byte chunks per K/V row
  constexpr int KU = BK * CH / kThreads;         // K chunks per thread per tile
  constexpr int VW = BK / 2;                     // 32-bit words per V^T row
  constexpr int VU = (BK / 2) * CH / kThreads;   // (key pair, chunk) units per thread
  static_assert(KU >= 1 && VU >= 1, "tile too small for the workgroup");

  __shared__ __attribute__((aligned(16))) u32x4 lds_k[2][BK * CH];
  __shared__ __attribute__((aligned(16))) uint32_t lds_vt[2][D * VW];

  // ---- work item: (batch, head, query tile) --------------------------------
  const int lin = blockIdx.x;
  int w = lin;
  if ((p.n_blocks & 7) == 0) w = (lin & 7) * (p.n_blocks >> 3) + (lin >> 3);
  const int bh = w / p.n_qtiles;
  int qt = w - bh * p.n_qtiles;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // heaviest tiles first
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int q0 = qt * kBQ;

  const size_t rs = (size_t)p.H * D;  // elements between consecutive tokens
  const uint16_t* __restrict__ Qb = p.q + ((size_t)b * p.Nq * p.H + h) * D;
  const uint16_t* __restrict__ Kb = p.k + ((size_t)b * p.Nk * p.H + h) * D;
  const uint16_t* __restrict__ Vb = p.v + ((size_t)b * p.Nk * p.H + h) * D;
  uint16_t* __restrict__ Ob = p.o + ((size_t)b * p.Nq * p.H + h) * D;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int qw0 = q0 + wave * 32;  // first query row of this wave
  const int my_q = qw0 + ln;       // query row owned by this lane

  // ---- Q fragments (B operand of S^T), read once ---------------------------
  u32x4 qf[DK];
  if (my_q < p.Nq) {
    const uint16_t* qrow = Qb + (size_t)my_q * rs + 8 * hf;
#pragma unroll
    for (int i = 0; i < DK; ++i) qf[i] = *reinterpret_cast<const u32x4*>(qrow + 16 * i);
  } else {
#pragma unroll
    for (int i = 0; i < DK; ++i) qf[i] = u32x4{0, 0, 0, 0};
  }

  // ---- key tiles this query tile needs -------------------------------------
  const int n_ktiles_all = (p.Nk + BK - 1) / BK;
  int n_kt = n_ktiles_all;
  if (CAUSAL) {
    const int qmax = min(p.Nq, q0 + kBQ);  // one past the last visible query
    n_kt = min(n_ktiles_all, (qmax + BK - 1) / BK);
  }

  // ---- global -> register prefetch, register -> LDS store ------------------
  u32x4 kreg[KU];
  u32x4 vreg[VU][2];

  // V unit mapping: one wave instruction covers 8 chunks x (64/8) key pairs
  // when CH == 8, or 16 chunks x 4 key pairs when CH == 16, so every key row
  // is read as whole 128/256-byte segments.
  auto v_unit = [&](int it, int& kp, int& dc) {
    if constexpr (CH == 16) {
      dc = (lane & 7) | ((lane >> 5) << 3);
      kp = (it * kWaves + wave) * 4 + ((lane >> 3) & 3);
    } else {
      dc = lane & 7;
      kp = (it * kWaves + wave) * 8 + (lane >> 3);
    }
  };

  auto load_tile = [&](int j) {
    const int kbase = j * BK;
#pragma unroll
    for (int it = 0; it < KU; ++it) {
      const int u = it * kThreads + tid;
      const int key = u / CH, c = u % CH;
      const int kk = kbase + key;
      if (kk < p.Nk)
        kreg[it] = *reinterpret_cast<const u32x4*>(Kb + (size_t)kk * rs + c * 8);
      else
        kreg[it] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int it = 0; it < VU; ++it) {
      int kp, dc;
      v_unit(it, kp, dc);
      const int k0 = kbase + 2 * kp;
      vreg[it][0] = (k0 < p.Nk) ? *reinterpret_cast<const u32x4*>(Vb + (size_t)k0 * rs + dc * 8)
                                : u32x4{0, 0, 0, 0};
      vreg[it][1] = (k0 + 1 < p.Nk)
                        ? *reinterpret_cast<const u32x4*>(Vb + (size_t)(k0 + 1) * rs + dc * 8)
                        : u32x4{0, 0, 0, 0};
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < KU; ++it) {
      const int u = it * kThreads + tid;
      const int key = u / CH, c = u % CH;
      lds_k[buf][key * CH + (c ^ k_swz(key))] = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < VU; ++it) {
      int kp, dc;
      v_unit(it, kp, dc);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t a = vreg[it][0][i >> 1];
        const uint32_t bb = vreg[it][1][i >> 1];
        const uint32_t word = (i & 1) ? ((a >> 16) | (bb & 0xffff0000u))
                                      : ((a & 0xffffu) | (bb << 16));
        const int d = dc * 8 + i;
        lds_vt[buf][d * VW + (kp ^ (4 * vt_swz(d)))] = word;
      }
    }
  };

  // ---- running state -------------------------------------------------------
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY;  // running max of raw scores q.k
  float l_run = 0.f;        // this lane's part of the running row sum
  const float c = p.scale_log2;

  load_tile(0);
  store_tile(0);

  for (int j = 0; j < n_kt; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_kt) load_tile(j + 1);
    __syncthreads();

    const int k0 = j * BK;
    const bool active = !CAUSAL || k0 <= qw0 + 31;
    if (active) {
      // S^T = K . Q^T for 64 keys x 32 queries
      f32x16 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        const int key = kb * 32 + k_row_order(ln);
        const u32x4* krow = &lds_k[buf][key * CH];
        const int sw = k_swz(key);
#pragma unroll
        for (int i = 0; i < DK; ++i) s[kb] = O_::mfma(krow[(2 * i + hf) ^ sw], qf[i], s[kb]);
      }

      // mask only where the tile crosses the diagonal or the end of the keys
      const bool need_mask = (k0 + BK > p.Nk) || (CAUSAL && k0 + BK - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 16 * (r >> 3) + 8 * hf + (r & 7);
            const bool vis = key < p.Nk && (!CAUSAL || key <= my_q);
            s[kb][r] = vis ? s[kb][r] : -INFINITY;
          }
      }

      // online softmax
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2((m_run - m_new) * c);
      const float mc = m_new * c;
      float rsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(__builtin_fmaf(s[kb][r], c, -mc));
          s[kb][r] = e;
          rsum += e;
        }
      l_run = l_run * alpha + rsum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

      // P^T fragments: k-step ks covers keys 16*ks + 8*hf + 0..7
      u32x4 pf[PK];
#pragma unroll
      for (int ks = 0; ks < PK; ++ks) {
        const int kb = ks >> 1, r0 = 8 * (ks & 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) pf[ks][t] = O_::pack(s[kb][r0 + 2 * t], s[kb][r0 + 2 * t + 1]);
      }

      // O^T += V^T . P^T
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 32 + ln;
        const uint32_t* vrow = &lds_vt[buf][d * VW];
        const int sw = vt_swz(d);
#pragma unroll
        for (int ks = 0; ks < PK; ++ks) {
          const int g = 2 * ks + hf;
          const u32x4 a = *reinterpret_cast<const u32x4*>(vrow + 4 * (g ^ sw));
          o[db] = O_::mfma(a, pf[ks], o[db]);
        }
      }
    }

    if (j + 1 < n_kt) store_tile(buf ^ 1);
  }

  // ---- epilogue: O = O^T / l, LSE = scale*m + ln(l) ------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_q < p.Nq) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = Ob + (size_t)my_q * rs;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 w2;
        w2[0] = O_::pack(o[db][4 * a + 0] * inv, o[db][4 * a + 1] * inv);
        w2[1] = O_::pack(o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * a + 4 * hf) = w2;
      }
    if (hf == 0) {
      const float lse = m_run * p.scale + fast_log2(l_tot) * 0.69314718055994531f;
      p.lse[((size_t)b * p.H + h) * p.Nq + my_q] = lse;
    }
  }
}

}  // namespace mha
