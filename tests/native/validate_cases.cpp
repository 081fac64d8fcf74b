// Host-only driver for the C-ABI argument checks (mha_validate.hpp): runs a
// table of calls -- valid ones, each kind of invalid argument, and sizes at
// and past every limit, up to INT_MAX -- and compares each status with the
// contract in include/mha.h. Built with AddressSanitizer and
// UndefinedBehaviorSanitizer (non-recovering) by tests/test_validate_sanitizers.py,
// so an out-of-range read or a signed overflow in the checks ends the run.
// Pointers are fake addresses: the checks only compare them, never read
// through them.
#include "../../head_attention_mha_amd/csrc/mha_validate.hpp"

#include <climits>
#include <cstdio>
#include <limits>

using namespace mha_host;

namespace {

int g_fail = 0, g_run = 0;

void expect(const char* what, mha_status_t got, mha_status_t want) {
  ++g_run;
  if (got != want) {
    ++g_fail;
    std::printf("FAIL %s: got %d want %d\n", what, (int)got, (int)want);
  }
}

// Disjoint, 256-byte aligned fake buffers, 2^40 bytes apart.
void* buf(int i) { return reinterpret_cast<void*>((uintptr_t)(i + 1) << 40); }
float* fbuf(int i) { return static_cast<float*>(buf(i)); }

mha_status_t fwd(int B, int H, int Nq, int Nk, int d, int causal = 1, float scale = 0.125f,
                 int dtype = MHA_DTYPE_BF16, bool* empty = nullptr) {
  bool e = false;
  return validate_fwd(buf(0), buf(1), buf(2), buf(3), fbuf(4), B, H, Nq, Nk, d, causal, scale,
                      dtype, mha::kBQ, empty ? empty : &e);
}

void fwd_cases() {
  const float inf = std::numeric_limits<float>::infinity();
  const float nan = std::numeric_limits<float>::quiet_NaN();
  bool empty = false;
  expect("fwd valid", fwd(1, 8, 16384, 16384, 128, 1, 0.088f, MHA_DTYPE_BF16, &empty), MHA_OK);
  expect("fwd valid is not empty", empty ? MHA_ERR_INVALID_ARG : MHA_OK, MHA_OK);
  expect("fwd empty B", fwd(0, 8, 16, 16, 64, 0, 0.125f, MHA_DTYPE_FP16, &empty), MHA_OK);
  expect("fwd empty flagged", empty ? MHA_OK : MHA_ERR_INVALID_ARG, MHA_OK);
  expect("fwd empty Nq, Nk 0", fwd(2, 2, 0, 0, 64), MHA_OK);
  expect("fwd Nk 0 with rows", fwd(1, 1, 4, 0, 64), MHA_ERR_INVALID_ARG);
  expect("fwd negative B", fwd(-1, 1, 1, 1, 64), MHA_ERR_INVALID_ARG);
  expect("fwd negative H", fwd(1, -1, 1, 1, 64), MHA_ERR_INVALID_ARG);
  expect("fwd negative Nq", fwd(1, 1, -5, 1, 64), MHA_ERR_INVALID_ARG);
  expect("fwd negative Nk", fwd(1, 1, 1, INT_MIN, 64), MHA_ERR_INVALID_ARG);
  expect("fwd causal 2", fwd(1, 1, 1, 1, 64, 2), MHA_ERR_INVALID_ARG);
  expect("fwd causal -1", fwd(1, 1, 1, 1, 64, -1), MHA_ERR_INVALID_ARG);
  expect("fwd dtype 7", fwd(1, 1, 1, 1, 64, 0, 0.125f, 7), MHA_ERR_INVALID_ARG);
  expect("fwd scale nan", fwd(1, 1, 1, 1, 64, 0, nan), MHA_ERR_INVALID_ARG);
  expect("fwd scale inf", fwd(1, 1, 1, 1, 64, 0, inf), MHA_ERR_INVALID_ARG);
  expect("fwd scale 0", fwd(1, 1, 1, 1, 64, 0, 0.f), MHA_ERR_INVALID_ARG);
  expect("fwd scale < 0", fwd(1, 1, 1, 1, 64, 0, -0.125f), MHA_ERR_INVALID_ARG);
  expect("fwd d 96", fwd(1, 1, 1, 1, 96), MHA_ERR_UNSUPPORTED);
  expect("fwd d 0", fwd(1, 1, 1, 1, 0), MHA_ERR_INVALID_ARG);
  expect("fwd d -64", fwd(1, 1, 1, 1, -64), MHA_ERR_INVALID_ARG);
  expect("fwd d INT_MAX", fwd(1, 1, 1, 1, INT_MAX), MHA_ERR_UNSUPPORTED);
  // token rows of H*d elements: at most 2^23 (32-bit offsets within a tile)
  expect("fwd H*d = 2^23", fwd(1, 65536, 1, 1, 128), MHA_OK);
  expect("fwd H*d > 2^23", fwd(1, 65537, 1, 1, 128), MHA_ERR_INVALID_ARG);
  expect("fwd H INT_MAX", fwd(1, INT_MAX, 1, 1, 128), MHA_ERR_INVALID_ARG);
  // grids of 2^31 workgroups or more
  expect("fwd grid 2^31 - 1 rows ok", fwd(1, 1, INT_MAX, 1, 64), MHA_OK);
  expect("fwd grid too large", fwd(INT_MAX, 1, INT_MAX, 1, 64), MHA_ERR_INVALID_ARG);
  expect("fwd all sizes INT_MAX", fwd(INT_MAX, INT_MAX, INT_MAX, INT_MAX, 64), MHA_ERR_INVALID_ARG);
  expect("fwd B, Nq INT_MAX, H*d at its limit", fwd(INT_MAX, 65536, INT_MAX, INT_MAX, 128),
         MHA_ERR_INVALID_ARG);
  expect("fwd B*H*Nq*d past 2^64", fwd(INT_MAX, 32768, INT_MAX, INT_MAX, 128), MHA_ERR_INVALID_ARG);
  bool e = false;
  // pointers
  expect("fwd null q", validate_fwd(nullptr, buf(1), buf(2), buf(3), fbuf(4), 1, 1, 4, 4, 64, 0,
                                    0.1f, 0, mha::kBQ, &e), MHA_ERR_INVALID_ARG);
  expect("fwd null lse", validate_fwd(buf(0), buf(1), buf(2), buf(3), nullptr, 1, 1, 4, 4, 64, 0,
                                      0.1f, 0, mha::kBQ, &e), MHA_ERR_INVALID_ARG);
  expect("fwd nulls on empty", validate_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 4,
                                            4, 64, 0, 0.1f, 0, mha::kBQ, &e), MHA_OK);
  char* base = static_cast<char*>(buf(0));
  expect("fwd misaligned k", validate_fwd(buf(0), base + (1LL << 40) + 8, buf(2), buf(3), fbuf(4),
                                          1, 1, 4, 4, 64, 0, 0.1f, 0, mha::kBQ, &e),
         MHA_ERR_INVALID_ARG);
  expect("fwd misaligned lse", validate_fwd(buf(0), buf(1), buf(2), buf(3),
                                            reinterpret_cast<float*>(base + (4LL << 40) + 2), 1, 1,
                                            4, 4, 64, 0, 0.1f, 0, mha::kBQ, &e),
         MHA_ERR_INVALID_ARG);
  expect("fwd o aliases q", validate_fwd(buf(0), buf(1), buf(2), buf(0), fbuf(4), 1, 1, 4, 4, 64,
                                         0, 0.1f, 0, mha::kBQ, &e), MHA_ERR_INVALID_ARG);
  // lse starts inside o's last bytes: o = 1*4*1*64*2 = 512 bytes
  expect("fwd lse overlaps o", validate_fwd(buf(0), buf(1), buf(2), buf(3),
                                            reinterpret_cast<float*>(base + (3LL << 40) + 496), 1,
                                            1, 4, 4, 64, 0, 0.1f, 0, mha::kBQ, &e),
         MHA_ERR_INVALID_ARG);
  expect("fwd lse right after o", validate_fwd(buf(0), buf(1), buf(2), buf(3),
                                               reinterpret_cast<float*>(base + (3LL << 40) + 512),
                                               1, 1, 4, 4, 64, 0, 0.1f, 0, mha::kBQ, &e),
         MHA_OK);
}

void split_cases() {
  bool e = false;
  auto sp = [&](int B, int H, int Nq, int Nk, int d, int n) {
    return validate_splitkv(buf(0), buf(1), buf(2), buf(3), fbuf(4), B, H, Nq, Nk, d, 0, 0.1f,
                            n, fbuf(5), fbuf(6), MHA_DTYPE_FP16, &e);
  };
  expect("split valid", sp(1, 32, 1, 32768, 128, 64), MHA_OK);
  expect("split 0 splits", sp(1, 1, 1, 16, 64, 0), MHA_ERR_INVALID_ARG);
  expect("split 257 splits", sp(1, 1, 1, 16, 64, 257), MHA_ERR_INVALID_ARG);
  expect("split Nq 9", sp(1, 1, 9, 16, 64, 1), MHA_ERR_UNSUPPORTED);
  expect("split Nk INT_MAX", sp(1, 1, 1, INT_MAX, 64, 256), MHA_ERR_INVALID_ARG);
  expect("split B*H*splits too large", sp(INT_MAX, 1024, 1, 16, 64, 256), MHA_ERR_INVALID_ARG);
  expect("split null workspace",
         validate_splitkv(buf(0), buf(1), buf(2), buf(3), fbuf(4), 1, 1, 1, 16, 64, 0, 0.1f, 2,
                          nullptr, fbuf(6), MHA_DTYPE_FP16, &e), MHA_ERR_INVALID_ARG);
  expect("split workspace aliases k",
         validate_splitkv(buf(0), buf(1), buf(2), buf(3), fbuf(4), 1, 1, 1, 16, 64, 0, 0.1f, 2,
                          fbuf(1), fbuf(6), MHA_DTYPE_FP16, &e), MHA_ERR_INVALID_ARG);
  expect("split H*d > 2^23", sp(1, 65537, 1, 16, 128, 1), MHA_ERR_INVALID_ARG);

  // the no-allocation variant: its workspace must fit the fixed scratch
  auto na = [&](int B, int H, int Nq, int Nk, int d, int n, size_t cap) {
    return validate_splitkv_noalloc(buf(0), buf(1), buf(2), buf(3), fbuf(4), B, H, Nq, Nk, d, 0,
                                    0.1f, n, MHA_DTYPE_BF16, cap, &e);
  };
  const size_t cap = 16u << 20;
  expect("noalloc decode fits", na(1, 32, 1, 32768, 128, 64, cap), MHA_OK);
  // 63 splits x 512 rows x 129 floats fits in 16 MiB, 64 do not
  expect("noalloc 63 splits fit", na(1, 64, 8, 256, 128, 63, cap), MHA_OK);
  expect("noalloc 64 splits too large", na(1, 64, 8, 256, 128, 64, cap), MHA_ERR_SCRATCH_TOO_SMALL);
  // exactly at the capacity: o_part 256 bytes (padded), lse_part 256 bytes
  expect("noalloc exactly at capacity", na(1, 1, 1, 16, 64, 1, 256 + 4), MHA_OK);
  expect("noalloc one byte short", na(1, 1, 1, 16, 64, 1, 256 + 3), MHA_ERR_SCRATCH_TOO_SMALL);
  expect("noalloc checks the arguments first", na(1, 1, 9, 16, 64, 1, cap), MHA_ERR_UNSUPPORTED);
  expect("noalloc bad splits", na(1, 1, 1, 16, 64, 0, cap), MHA_ERR_INVALID_ARG);
  expect("noalloc empty", na(0, 1, 1, 16, 64, 4, 0), MHA_OK);
  expect("noalloc huge", na(INT_MAX, INT_MAX, 8, INT_MAX, 128, 256, cap), MHA_ERR_INVALID_ARG);
}

void bwd_cases() {
  bool eq = false, ek = false;
  auto bw = [&](int B, int H, int Nq, int Nk, int d) {
    return validate_bwd(buf(0), buf(1), buf(2), buf(3), buf(4), fbuf(5), buf(6), buf(7), buf(8),
                        fbuf(9), B, H, Nq, Nk, d, 1, 0.1f, MHA_DTYPE_BF16, &eq, &ek);
  };
  expect("bwd valid", bw(1, 8, 16384, 16384, 128), MHA_OK);
  expect("bwd empty", bw(0, 8, 16, 16, 64), MHA_OK);
  expect("bwd keys only", bw(1, 1, 0, 16, 64), MHA_OK);
  expect("bwd Nk 0 with rows", bw(1, 1, 16, 0, 64), MHA_ERR_INVALID_ARG);
  expect("bwd d 32", bw(1, 1, 16, 16, 32), MHA_ERR_UNSUPPORTED);
  expect("bwd H*d > 2^23", bw(1, 65537, 1, 1, 128), MHA_ERR_INVALID_ARG);
  expect("bwd grid too large", bw(INT_MAX, 2, INT_MAX, INT_MAX, 64), MHA_ERR_INVALID_ARG);
  expect("bwd all INT_MAX", bw(INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128), MHA_ERR_INVALID_ARG);
  expect("bwd dq aliases dk",
         validate_bwd(buf(0), buf(1), buf(2), buf(3), buf(4), fbuf(5), buf(6), buf(6), buf(8),
                      fbuf(9), 1, 1, 4, 4, 64, 0, 0.1f, 0, &eq, &ek), MHA_ERR_INVALID_ARG);
}

void kl_cases() {
  bool e = false;
  auto k = [&](int B, int H, int Nq, int Nk, int d) {
    return validate_kl(buf(0), buf(1), buf(2), buf(3), fbuf(4), fbuf(5), fbuf(6), B, H, Nq, Nk,
                       d, 1, 0.1f, MHA_DTYPE_BF16, &e);
  };
  expect("kl valid", k(1, 8, 16384, 16384, 128), MHA_OK);
  expect("kl H*d > 2^23", k(1, 65537, 1, 1, 128), MHA_ERR_INVALID_ARG);
  expect("kl grid too large", k(INT_MAX, 4, INT_MAX, 1, 64), MHA_ERR_INVALID_ARG);
  expect("kl all INT_MAX", k(INT_MAX, INT_MAX, INT_MAX, INT_MAX, 64), MHA_ERR_INVALID_ARG);
  expect("kl lse2 aliases kl",
         validate_kl(buf(0), buf(1), buf(2), buf(3), fbuf(4), fbuf(5), fbuf(4), 1, 1, 4, 4, 64, 0,
                     0.1f, 0, &e), MHA_ERR_INVALID_ARG);
}

void proj_cases() {
  bool e = false;
  auto pr = [&](int B, int Nq, int H, int d, int E) {
    return validate_proj(buf(0), buf(1), buf(2), buf(3), B, Nq, H, d, E, MHA_DTYPE_BF16, &e);
  };
  expect("proj valid", pr(1, 16384, 8, 128, 1024), MHA_OK);
  expect("proj K = 2^23", pr(1, 16, 65536, 128, 64), MHA_OK);
  expect("proj K > 2^23", pr(1, 16, 65537, 128, 64), MHA_ERR_INVALID_ARG);
  expect("proj K not a multiple of 64", pr(1, 16, 1, 96, 64), MHA_ERR_UNSUPPORTED);
  expect("proj E not a multiple of 4", pr(1, 16, 1, 64, 66), MHA_ERR_UNSUPPORTED);
  expect("proj M too large", pr(INT_MAX, INT_MAX, 1, 64, 64), MHA_ERR_INVALID_ARG);
  expect("proj H*d overflows int", pr(1, 16, INT_MAX, INT_MAX, 64), MHA_ERR_INVALID_ARG);
  expect("proj all INT_MAX", pr(INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX), MHA_ERR_INVALID_ARG);
  expect("proj empty", pr(0, 16, 1, 64, 64), MHA_OK);
  expect("proj y aliases w", validate_proj(buf(0), buf(1), nullptr, buf(1), 1, 16, 1, 64, 64,
                                           MHA_DTYPE_FP16, &e), MHA_ERR_INVALID_ARG);
}

}  // namespace

int main() {
  fwd_cases();
  split_cases();
  bwd_cases();
  kl_cases();
  proj_cases();
  std::printf("%d of %d cases as the contract states\n", g_run - g_fail, g_run);
  return g_fail ? 1 : 0;
}
