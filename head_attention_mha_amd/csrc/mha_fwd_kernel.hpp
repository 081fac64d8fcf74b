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
//      alpha = exp(scale*(m_old - m_new)) when the max has grown;
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
// * K and V tiles are copied global -> LDS by buffer loads that write LDS
//   directly (no staging registers); rows past the end of the keys read as
//   zero through the buffer's range check, so the tail needs no branches.
//   The copy of tile j+1 is in flight while tile j is computed.
// * V stays row-major in LDS; the V^T operand of the P.V product comes from
//   gfx950 LDS transpose reads (ds_read_b64_tr_b16), two per MFMA.
// * LDS tiles are XOR-swizzled in 16-byte units so the MFMA operand reads
//   are free of bank conflicts.
// * The O rescale is deferred while a row's max stays within 2^8 (exp2
//   domain) of the max O and l were last scaled to; O/l and LSE are the same
//   in exact arithmetic, and the rescale then runs only when the max jumps.
// * At most 256 registers per lane, so two waves share each SIMD and one
//   wave's softmax overlaps the other's MFMAs.
// * The 1-D grid is remapped so that consecutive work items of one head land
//   on the same XCD (workgroups are dispatched round-robin over the 8 XCDs),
//   keeping a head's K/V in that XCD's L2; causal query tiles run heaviest
//   first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;  // query rows per workgroup
constexpr int kBK = 64;           // keys per tile
// The O rescale is deferred while a row's running max stays within 2^8 (in
// the exp2 domain) of the reference max the accumulators were scaled to.
constexpr float kDeferLog2 = 8.0f;

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
//  V, read by transpose reads: 16 lanes touch 4 consecutive rows x 32 bytes.
template <int D>
__device__ __forceinline__ int v_swz(int key) {
  const int t = key & 3;
  if constexpr (D == 128) return 4 * t + 2 * (t >> 1);
  else return 2 * t;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// gfx950 LDS transpose read of 4 x 16-bit values. Within each group of 16
// lanes, lane i receives element (i % 4) of the 8-byte rows addressed by
// lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)p));
  return __builtin_bit_cast(u32x2, r);
}

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

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mha_fwd_kernel(Params p) {
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

  __shared__ __attribute__((aligned(1024))) uint8_t lds_k0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v1[TILEB];

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
  const uint32_t row_bytes = (uint32_t)(rs * 2);

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

  // Per-lane source offsets of this wave's 1 KiB copies (same for every tile).
  uint32_t k_off[NCPW], v_off[NCPW];
#pragma unroll
  for (int it = 0; it < NCPW; ++it) {
    const int row = (it * kWaves + wave) * RPI + lane / CH;
    const int pc = lane % CH;  // physical chunk in LDS
    k_off[it] = row * row_bytes + 16 * (pc ^ k_swz<D>(row));
    v_off[it] = row * row_bytes + 16 * (pc ^ v_swz<D>(row));
  }

  // Issue the asynchronous global -> LDS copies of key tile j.
  auto issue = [&](int j, uint8_t* lk, uint8_t* lv) __attribute__((always_inline)) {
    const int kbase = j * BK;
    const int nvalid = min(BK, p.Nk - kbase);
    const uint32_t bytes = (uint32_t)(nvalid - 1) * row_bytes + ROWB;
    const auto rk = make_rsrc(Kb + (size_t)kbase * rs, bytes);
    const auto rv = make_rsrc(Vb + (size_t)kbase * rs, bytes);
#pragma unroll
    for (int it = 0; it < NCPW; ++it) {
      const int c = it * kWaves + wave;
      dma16(rk, lk + c * 1024, k_off[it]);
      dma16(rv, lv + c * 1024, v_off[it]);
    }
  };

  // ---- running state -------------------------------------------------------
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY;  // reference max (raw scores q.k) of o and l_run
  float l_run = 0.f;        // this lane's part of the row sum
  const float c = p.scale_log2;

  // Key tiles [0, jm) need no element mask for any row of this workgroup;
  // [jm, n_kt) may (the last, partial tile; the tiles crossing the causal
  // diagonal of rows q0 .. q0+BQ-1).
  int jm = (p.Nk % BK) ? p.Nk / BK : n_ktiles_all;
  if (CAUSAL) jm = min(jm, (q0 + 1) / BK);
  jm = min(jm, n_kt);

  auto compute = [&](int j, const uint8_t* lk, const uint8_t* lv, bool masked)
                     __attribute__((always_inline)) {
    const int k0 = j * BK;
    if (CAUSAL && k0 > qw0 + 31) return;  // tile wholly past this wave's rows

    // S^T = K . Q^T for 64 keys x 32 queries: two independent accumulation
    // chains (one per 32-key block), interleaved per k-step
    f32x16 s[KB];
    const uint8_t* krow[KB];
    int ksw[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const int key = kb * 32 + k_row_order(ln);
      krow[kb] = lk + key * ROWB;
      ksw[kb] = k_swz<D>(key);
    }
#pragma unroll
    for (int i = 0; i < DK; ++i)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        s[kb] = O_::mfma(*reinterpret_cast<const u32x4*>(krow[kb] + 16 * ((2 * i + hf) ^ ksw[kb])),
                         qf[i], s[kb]);

    // mask only where the tile crosses the diagonal or the end of the keys;
    // the empty asm keeps the compiler from turning this rarely taken,
    // wave-uniform branch into selects executed on every tile
    if (masked) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 16 * (r >> 3) + 8 * hf + (r & 7);
          const bool vis = key < p.Nk && (!CAUSAL || key <= my_q);
          s[kb][r] = vis ? s[kb][r] : -INFINITY;
        }
    }

    // online softmax; the rescale of O and l is deferred while the tile max
    // stays within kDeferLog2 of the reference max
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
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
    const float mc = m_run * c;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], c, -mc));

    // P^T fragments: k-step ks covers keys 16*ks + 8*hf + 0..7.
    u32x4 pf[PK];
    float rsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < PK; ++ks) {
      const int kb = ks >> 1, r0 = 8 * (ks & 1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        pf[ks][t] = O_::pack(s[kb][r0 + 2 * t], s[kb][r0 + 2 * t + 1]);
        rsum = O_::sum2(pf[ks][t], s[kb][r0 + 2 * t], s[kb][r0 + 2 * t + 1], rsum);
      }
    }
    l_run += rsum;

    // O^T += V^T . P^T; V^T fragments by transpose reads of row-major V. The
    // DB accumulators are independent, so they are interleaved per k-step.
    const int grp = lane >> 4, li = lane & 15;
#pragma unroll
    for (int ks = 0; ks < PK; ++ks) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int dch = 4 * db + 2 * (grp & 1) + ((li & 3) >> 1);  // 16-byte chunk of d
        const int dsub = 8 * (li & 1);                              // byte offset in it
        u32x4 a;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int key = ks * 16 + 8 * (grp >> 1) + 4 * r + (li >> 2);
          const u32x2 t = lds_read_tr16(lv + key * ROWB + 16 * (dch ^ v_swz<D>(key)) + dsub);
          a[2 * r] = t[0];
          a[2 * r + 1] = t[1];
        }
        o[db] = O_::mfma(a, pf[ks], o[db]);
      }
    }
  };

  // ---- main loop: double-buffered, one barrier per key tile ----------------
  // step: wait for tile j in buffer `buf`, start the copy of tile j+1 into
  // the other buffer (last read by tile j-1, which every wave has finished
  // once past the barrier), then compute tile j.
  auto step = [&](int j, auto buf) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile j landed
    __syncthreads();
    if constexpr (decltype(buf)::value == 0) {
      if (j + 1 < n_kt) issue(j + 1, lds_k1, lds_v1);
      compute(j, lds_k0, lds_v0, j >= jm);
    } else {
      if (j + 1 < n_kt) issue(j + 1, lds_k0, lds_v0);
      compute(j, lds_k1, lds_v1, j >= jm);
    }
  };
  issue(0, lds_k0, lds_v0);
  for (int j = 0; j < n_kt; j += 2) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 < n_kt) step(j + 1, std::integral_constant<int, 1>{});
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
