// Split-KV attention forward for few query rows (decode) on gfx950.
//
// With Nq small (one new token per sequence when decoding, or a handful), the
// forward has almost no arithmetic per byte: every key and value row is read
// once and used for at most 8 dot products. The work is HBM-bound, so it is
// spread over the keys instead of the queries ("StreamKL", Methodology
// section 3: when NQ is small, keys are split across thread blocks and the
// partial results merged): workgroup (b, h, s) owns keys [s*L, (s+1)*L),
// computes the softmax-normalised partial O_s and its LSE_s for every query
// row, and a second kernel merges the splits of a row with
//
//   LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
//
// which is the softmax over the union of the key sets (the LSE of the
// "StreamKL" online formulation, Methodology section 1, taken over blocks of
// keys instead of single keys).
//
// The partial kernel uses the vector ALU, not MFMA: a key row of d 16-bit
// values is spread over d/8 lanes (16 bytes each, one coalesced row segment),
// so a wave reads 4 (d = 128) or 8 (d = 64) rows per load instruction; the
// per-row dot products are finished with DPP adds inside each group of d/8
// lanes. Each lane group keeps its own online-softmax state (running max m,
// sum l, its d/8 output channels) over the keys it visits; the 16 or 32
// groups of a workgroup are merged through LDS at the end.
#pragma once

#include "mha_fwd_kernel.hpp"

namespace mha {

struct SplitParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* o_part;    // [n_splits, B, H, Nq, d] fp32: normalised partial outputs
  float* lse_part;  // [n_splits, B, H, Nq] fp32: partial LSEs (-inf: no visible key)
  int B, H, Nq, Nk;
  float scale;       // softmax scale (> 0)
  float scale_log2;  // scale * log2(e)
  int n_splits;
  int split_len;     // keys per split (a multiple of the workgroup step)
};

namespace split {

// kWaves, kThreads and kMaxNq are in mha_tiles.hpp
constexpr float kLn2 = 0.69314718055994531f;

// x summed over the 2^LOG lanes of its group (groups of 8 or 16 lanes), in
// every lane of the group: DPP swaps within quads, then the half-row and row
// mirrors.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
template <int LOG>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_mov<0xB1>(x);                      // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);                      // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);                     // row_half_mirror
  if constexpr (LOG == 4) x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

template <typename T>
__device__ __forceinline__ void unpack8(const u32x4 w, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = w[i];
    if constexpr (std::is_same<T, BF16>::value) {
      f[2 * i] = __builtin_bit_cast(float, x << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, x & 0xffff0000u);
    } else {
      const f32x2 y = __builtin_convertvector(__builtin_bit_cast(f16x2, x), f32x2);
      f[2 * i] = y[0];
      f[2 * i + 1] = y[1];
    }
  }
}

}  // namespace split

// ---- partial outputs of one split ----------------------------------------------
// Workgroup lin -> (bh, s) = (lin / n_splits, lin % n_splits). Lane group
// g = tid / LPR (16 or 32 groups) handles keys k_beg + it*STEP + g, one per
// iteration, KB iterations per block (scores of a block first, then one
// max/rescale per block).
template <typename T, int D, int NQ, bool CAUSAL>
__global__ __launch_bounds__(split::kThreads) void mha_split_partial_kernel(SplitParams p) {
  constexpr int LPR = D / 8;                    // lanes per key row
  constexpr int LOG = D == 128 ? 4 : 3;
  constexpr int NG = split::kThreads / LPR;     // lane groups (keys per step)
  constexpr int KB = NQ <= 2 ? 8 : 4;           // keys per group per block
  const int tid = threadIdx.x;
  const int g = tid / LPR;
  const int part = tid % LPR;                   // this lane's 8 channels: 8*part .. +7
  const int bh = blockIdx.x / p.n_splits;
  const int sp = blockIdx.x - bh * p.n_splits;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int k_beg = sp * p.split_len;
  const int k_end = min(p.Nk, k_beg + p.split_len);
  const size_t rs = (size_t)p.H * D;
  const size_t qo = ((size_t)b * p.Nq * p.H + h) * D;
  const size_t kvo = ((size_t)b * p.Nk * p.H + h) * D;
  const float c = p.scale_log2;

  // this lane's 8 channels of every query row, scaled into the log2 domain
  float qv[NQ][8];
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    if (n < p.Nq) {
      float f[8];
      split::unpack8<T>(*reinterpret_cast<const u32x4*>(p.q + qo + (size_t)n * rs + 8 * part), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[n][i] = f[i] * c;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[n][i] = 0.f;
    }
  }
  float m[NQ], l[NQ], acc[NQ][8];
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    m[n] = -__builtin_inff();
    l[n] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[n][i] = 0.f;
  }

  const uint16_t* kbase = p.k + kvo + 8 * part;
  const uint16_t* vbase = p.v + kvo + 8 * part;
  for (int k0 = k_beg; k0 < k_end; k0 += NG * KB) {
    // loads of this block (rows past k_end are not read)
    u32x4 kr[KB], vr[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int key = k0 + j * NG + g;
      if (key < k_end) {
        kr[j] = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * rs);
        vr[j] = *reinterpret_cast<const u32x4*>(vbase + (size_t)key * rs);
      } else {
        kr[j] = vr[j] = u32x4{0, 0, 0, 0};
      }
    }
    // scores (log2 domain) of the block's keys for every query row
    float s[KB][NQ];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      float kf[8];
      split::unpack8<T>(kr[j], kf);
      const int key = k0 + j * NG + g;
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) x = __builtin_fmaf(qv[n][i], kf[i], x);
        x = split::group_sum<LOG>(x);
        const bool vis = key < k_end && (!CAUSAL || key <= n);
        s[j][n] = vis ? x : -__builtin_inff();
      }
    }
    // one max and rescale per block, then P V
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      float mb = s[0][n];
#pragma unroll
      for (int j = 1; j < KB; ++j) mb = fmaxf(mb, s[j][n]);
      const float mn = fmaxf(m[n], mb);
      // reference max; 0 while nothing is visible, so that the weights below
      // are exp2(-inf) = 0 instead of exp2(-inf + inf)
      const float mref = mn == -__builtin_inff() ? 0.f : mn;
      const float alpha = fast_exp2(m[n] - mref);
      m[n] = mn;
      l[n] *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[n][i] *= alpha;
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const float pj = fast_exp2(s[j][n] - mref);
        l[n] += pj;
        float vf[8];
        split::unpack8<T>(vr[j], vf);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[n][i] = __builtin_fmaf(pj, vf[i], acc[n][i]);
      }
    }
  }

  // merge the NG lane groups: (m, l) per group and query, then the channels
  __shared__ float sm_m[split::kMaxNq][NG];
  __shared__ float sm_l[split::kMaxNq][NG];
  __shared__ float sm_o[NG][D + 4];
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    if (part == 0) {
      sm_m[n][g] = m[n];
      sm_l[n][g] = l[n];
    }
  }
  __syncthreads();
  const size_t row_base = ((size_t)sp * p.B * p.H + bh) * p.Nq;  // [s][b][h][n] row index
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    if (n >= p.Nq) break;
    // every thread finds the workgroup max and this group's weight
    float M = -__builtin_inff();
    for (int t = 0; t < NG; ++t) M = fmaxf(M, sm_m[n][t]);
    const float wgt = M == -__builtin_inff() ? 0.f : fast_exp2(m[n] - M);
#pragma unroll
    for (int i = 0; i < 8; ++i) sm_o[g][8 * part + i] = acc[n][i] * wgt;
    __syncthreads();
    // thread t < D sums channel t over the groups
    if (tid < D) {
      float L = 0.f, O = 0.f;
      for (int t = 0; t < NG; ++t) {
        const float mt = sm_m[n][t];
        if (mt != -__builtin_inff()) L += sm_l[n][t] * fast_exp2(mt - M);
        O += sm_o[t][tid];
      }
      const size_t r = row_base + n;
      p.o_part[r * D + tid] = L > 0.f ? O / L : 0.f;
      if (tid == 0) p.lse_part[r] = L > 0.f ? (M + fast_log2(L)) * split::kLn2 : -__builtin_inff();
    }
    __syncthreads();
  }
}

// ---- merge of the splits ---------------------------------------------------------
// One workgroup per row r = (b*H + h)*Nq + n. The merge is a few dependent
// memory round trips on little data, so it is laid out for latency: thread
// (g, c) first issues the loads of channels 4c .. 4c+3 of its splits
// s = g + G*i (i < kPre), which do not depend on the weights; meanwhile
// thread t < n_splits reads LSE_t, the workgroup takes their maximum M and
// stores the weights w_s = exp(LSE_s - M) in LDS; then every thread adds
// w_s * O_s over its splits and the G partial sums are added through LDS.
// Empty splits have LSE = -inf and O = 0, weight 0.
template <typename T, int D>
__global__ __launch_bounds__(split::kThreads) void mha_split_merge_kernel(SplitParams p) {
  constexpr int TPR = D / 4;                   // channel threads per split group
  constexpr int G = split::kThreads / TPR;     // split groups
  constexpr int NW = split::kThreads / 64;
  constexpr int kPre = 8;                      // splits per group loaded up front
  constexpr float NEG_INF = -__builtin_inff();
  __shared__ float sm_w[split::kThreads];      // n_splits <= kThreads
  __shared__ float sm_max[NW];
  __shared__ float sm_l[G];
  __shared__ float sm_o[G][D];
  const long long r = blockIdx.x;
  const long long n_rows = (long long)p.B * p.H * p.Nq;
  const int n = p.n_splits;
  const int tid = threadIdx.x;
  const int g = tid / TPR;
  const int c4 = (tid - g * TPR) * 4;
  float4 x[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int s = g + G * i;
    x[i] = s < n ? *reinterpret_cast<const float4*>(p.o_part + (s * n_rows + r) * D + c4)
                 : float4{0.f, 0.f, 0.f, 0.f};
  }
  const float ls = tid < n ? p.lse_part[tid * n_rows + r] : NEG_INF;
  float M = ls;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((tid & 63) == 0) sm_max[tid >> 6] = M;
  __syncthreads();
  M = sm_max[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_max[w]);
  if (tid < n) sm_w[tid] = ls == NEG_INF ? 0.f : __expf(ls - M);
  __syncthreads();
  float L = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int s = g + G * i;
    if (s < n) {
      const float w = sm_w[s];
      L += w;
      o[0] = __builtin_fmaf(w, x[i].x, o[0]);
      o[1] = __builtin_fmaf(w, x[i].y, o[1]);
      o[2] = __builtin_fmaf(w, x[i].z, o[2]);
      o[3] = __builtin_fmaf(w, x[i].w, o[3]);
    }
  }
  for (int s = g + G * kPre; s < n; s += G) {
    const float w = sm_w[s];
    L += w;
    const float4 y = *reinterpret_cast<const float4*>(p.o_part + (s * n_rows + r) * D + c4);
    o[0] = __builtin_fmaf(w, y.x, o[0]);
    o[1] = __builtin_fmaf(w, y.y, o[1]);
    o[2] = __builtin_fmaf(w, y.z, o[2]);
    o[3] = __builtin_fmaf(w, y.w, o[3]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) sm_o[g][c4 + i] = o[i];
  if (c4 == 0) sm_l[g] = L;
  __syncthreads();
  if (g != 0) return;
  L = 0.f;
#pragma unroll
  for (int t = 0; t < G; ++t) L += sm_l[t];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = 0.f;
#pragma unroll
    for (int t = 0; t < G; ++t) v += sm_o[t][c4 + i];
    o[i] = v;
  }
  const float inv = 1.f / L;
  // O is laid out [b][n][h]: r = bh*Nq + n
  const long long bh = r / p.Nq;
  const int nq = (int)(r - bh * p.Nq);
  const int b = (int)(bh / p.H), h = (int)(bh - (long long)b * p.H);
  uint16_t* dst = p.o + (((size_t)b * p.Nq + nq) * p.H + h) * D + c4;
  u32x2 w2;
  w2[0] = Ops<T>::pack(o[0] * inv, o[1] * inv);
  w2[1] = Ops<T>::pack(o[2] * inv, o[3] * inv);
  *reinterpret_cast<u32x2*>(dst) = w2;
  if (c4 == 0) p.lse[r] = M + logf(L);
}

}  // namespace mha
