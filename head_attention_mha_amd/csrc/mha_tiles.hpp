// Workgroup shapes and tile sizes of the kernels: plain constants, shared by
// the kernels and by the host-side argument checks (which need the number
// of workgroups a call launches and the tile row counts that bound the
// kernels' 32-bit buffer offsets). No HIP dependency.
#pragma once

namespace mha {

// fused forward (mha_fwd_kernel): two groups of four waves, one wave of each
// per SIMD
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;  // query rows per workgroup (32 per wave)
constexpr int kBK = 64;           // keys per tile

namespace split {  // split-over-keys forward (partial and merge kernels)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxNq = 8;         // query rows per (b, h) the partial kernel handles
constexpr int kMaxSplits = 256;   // the merge reads one partial LSE per thread
constexpr int kSplitAlign = 256;  // keys per split are a multiple of this
static_assert(kMaxSplits <= kThreads, "the merge reads one LSE per thread");
}  // namespace split

namespace kl {  // fused attention-KL forward
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;  // query rows per workgroup
constexpr int kBK = 64;           // keys per tile
}  // namespace kl

namespace bwd {  // backward: D, dQ and dK/dV kernels
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;   // query rows per dq workgroup
constexpr int kBKV = 32 * kWaves;  // keys per dkdv workgroup
constexpr int kBK = 64;            // keys per tile streamed by dq
constexpr int kBQt = 32;           // queries per tile streamed by dkdv
}  // namespace bwd

namespace proj {  // output projection GEMM
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 256;  // output features per workgroup
constexpr int kBM = 256;  // tokens per workgroup
constexpr int kBK = 64;   // K per stage
}  // namespace proj

}  // namespace mha
