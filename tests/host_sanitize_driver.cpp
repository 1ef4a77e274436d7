// Drives the host side of the C ABI (ra_host.cpp) without a GPU, for a
// build with AddressSanitizer and UndefinedBehaviorSanitizer: the planner
// at the shapes of every workload, argument validation, the key-split and
// workspace helpers, and the forward / backward / feedforward entry points
// up to the launch.  The launchers are stubs that record the parameters the
// host derived, so that the grid sizes can be checked as well.  Fake device
// pointers are never dereferenced.  Exit status 0 = every check passed.

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "ra_attn.h"
#include "ra_decode.h"
#include "ra_internal.h"

namespace ra {
static FwdParams g_fwd;
static BwdParams g_bwd;
static int g_launches = 0;
int launch_fwd(const FwdParams& p, Dtype, int, int64_t, void*, char*, int) {
  g_fwd = p;
  ++g_launches;
  return 0;
}
int launch_bwd(const BwdParams& p, Dtype, int, void*, char*, int) {
  g_bwd = p;
  ++g_launches;
  return 0;
}
int launch_ffn(const FfnParams&, void*, char*, int) {
  ++g_launches;
  return 0;
}
static DecParams g_dec;
static int g_dec_nq = 0;
int launch_decode(const DecParams& p, Dtype, int, int nq, void*, char*, int) {
  g_dec = p;
  g_dec_nq = nq;
  ++g_launches;
  return 0;
}
int fwd_scratch(void** ptr, char*, int) {
  *ptr = reinterpret_cast<void*>(static_cast<uintptr_t>(1) << 24);
  return 0;
}
}  // namespace ra

static int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::printf("FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, \
                  ra_last_error());                                   \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

struct Shape {
  int64_t B, Lq, H, D;
  int32_t N, r;
  int64_t c, qc, kc;
};

int main() {
  // A fake, 256-byte aligned device address.
  char* const P = reinterpret_cast<char*>(static_cast<uintptr_t>(1) << 20);
  // The workloads' shapes (tiny, small causal, 7B share, packed documents,
  // 65B share) and a striped-like small one.
  const Shape shapes[] = {{1, 64, 2, 64, 4, 0, 0, 32, 32},
                          {1, 1024, 8, 128, 8, 7, 1, 512, 512},
                          {1, 32768, 32, 128, 16, 15, 1, 2048, 2048},
                          {4, 2048, 32, 128, 8, 3, 1, 512, 512},
                          {1, 16384, 64, 128, 256, 128, 16384, 512, 512}};
  for (const Shape& s : shapes) {
    // Planner: exactly sized host buffers, so any overrun is caught.
    std::vector<int32_t> order(s.N);
    std::vector<uint8_t> run((size_t)s.N * (s.Lq / s.qc) * (s.Lq / s.kc));
    int64_t n_run = -1;
    for (int place = 0; place < 2; ++place) {
      const int64_t c = place ? (s.c ? 1 : 0) : s.c;
      CHECK(ra_blockwise_plan_placed(c, s.qc, s.kc, s.Lq, s.N, s.r, (ra_placement_t)place,
                                     order.data(), run.data(), &n_run) == RA_OK);
      CHECK(n_run >= 1 && n_run <= (int64_t)run.size());
    }
    // Forward through every entry point, unsplit and split.
    const int64_t tiles = (s.Lq + 255) / 256;
    for (int32_t splits : {1, 2, 8, 64}) {
      const int64_t ws = ra_blockwise_attn_fwd_split_workspace_bytes(s.B, s.Lq, s.H, s.D, splits);
      CHECK(ws == (splits > 1 ? (int64_t)splits * s.B * s.H * s.Lq * (s.D + 2) * 4 : 0));
      ra::g_fwd = ra::FwdParams{};
      CHECK(ra_blockwise_attn_fwd_split(P, P, P, nullptr, s.c, s.qc, s.kc, s.N, s.r,
                                        RA_PLACE_CONTIGUOUS, s.B, s.Lq, s.H, s.D, RA_BF16, P,
                                        reinterpret_cast<float*>(P), nullptr, splits,
                                        splits > 1 ? P : nullptr, ws, nullptr) == RA_OK);
      // One workgroup per run: at least one per query tile, at most splits.
      CHECK(ra::g_fwd.n_wg >= s.B * s.H * tiles && ra::g_fwd.n_wg <= s.B * s.H * tiles * splits);
      CHECK(splits == 1 || ra::g_fwd.n_wg == s.B * s.H * ra::g_fwd.split_wgs);
      CHECK(ra::g_fwd.key_splits == splits);
      CHECK((ra::g_fwd.part_o != nullptr) == (splits > 1));
      if (splits > 1) {
        CHECK(reinterpret_cast<char*>(ra::g_fwd.part_ml) ==
              P + (int64_t)splits * s.B * s.H * s.Lq * s.D * 4);
        // one byte short
        CHECK(ra_blockwise_attn_fwd_split(P, P, P, nullptr, s.c, s.qc, s.kc, s.N, s.r,
                                          RA_PLACE_CONTIGUOUS, s.B, s.Lq, s.H, s.D, RA_BF16, P,
                                          reinterpret_cast<float*>(P), nullptr, splits, P, ws - 1,
                                          nullptr) == RA_E_INVALID);
      }
      // The no-allocation forward: its own scratch when the partials fit
      // 64 MiB, a refusal otherwise.
      ra::g_fwd = ra::FwdParams{};
      const ra_status_t na = ra_blockwise_attn_fwd_split_noalloc(
          P, P, P, nullptr, s.c, s.qc, s.kc, s.N, s.r, RA_PLACE_CONTIGUOUS, s.B, s.Lq, s.H, s.D,
          RA_BF16, P, reinterpret_cast<float*>(P), nullptr, splits, nullptr);
      if (ws <= ra::kFwdScratchBytes) {
        CHECK(na == RA_OK);
        CHECK(ra::g_fwd.key_splits == splits);
        CHECK(splits == 1 || ra::g_fwd.part_o == reinterpret_cast<float*>(
                                 static_cast<uintptr_t>(1) << 24));
      } else {
        CHECK(na == RA_E_UNSUPPORTED);
      }
      const int64_t bws = ra_blockwise_attn_bwd_split_workspace_bytes(s.B, s.Lq, s.H, s.D, splits);
      float* const F = reinterpret_cast<float*>(P);
      CHECK(ra_blockwise_attn_bwd_split(P, P, P, nullptr, s.c, s.qc, s.kc, s.N, s.r,
                                        RA_PLACE_CONTIGUOUS, s.B, s.Lq, s.H, s.D, RA_BF16, P, F,
                                        P, F, F, F, F, splits, splits > 1 ? P : nullptr, bws,
                                        nullptr) == RA_OK);
      CHECK(ra::g_bwd.f.n_wg >= s.B * s.H * tiles && ra::g_bwd.f.n_wg <= s.B * s.H * tiles * splits);
      CHECK(splits == 1 || ra::g_bwd.f.n_wg == s.B * s.H * ra::g_bwd.f.split_wgs);
      CHECK(ra::g_bwd.n_wg_kv == s.B * s.H * ((s.N * s.Lq + 255) / 256));
      CHECK((ra::g_bwd.dq_part != nullptr) == (splits > 1));
      // float32: the dq grid of 128-row tiles, dK/dV workgroups of 128 keys
      CHECK(ra_blockwise_attn_bwd_split(P, P, P, nullptr, s.c, s.qc, s.kc, s.N, s.r,
                                        RA_PLACE_CONTIGUOUS, s.B, s.Lq, s.H, s.D, RA_F32, P, F,
                                        P, F, F, F, F, splits, splits > 1 ? P : nullptr, bws,
                                        nullptr) == RA_OK);
      const int64_t tiles32 = (s.Lq + 127) / 128;
      CHECK(ra::g_bwd.f.n_wg >= s.B * s.H * tiles32 &&
            ra::g_bwd.f.n_wg <= s.B * s.H * tiles32 * splits);
      CHECK(splits == 1 || ra::g_bwd.f.n_wg == s.B * s.H * ra::g_bwd.f.split_wgs);
      CHECK(ra::g_bwd.n_wg_kv == s.B * s.H * ((s.N * s.Lq + 127) / 128));
    }
    CHECK(ra_blockwise_attn_fwd(P, P, P, nullptr, s.c, s.qc, s.kc, s.N, s.r, s.B, s.Lq, s.H,
                                s.D, RA_BF16, P, reinterpret_cast<float*>(P), nullptr) == RA_OK);
    for (int32_t r : {0, s.N - 1})
      for (int place = 0; place < 2; ++place) {
        const int32_t k = ra_blockwise_attn_fwd_key_splits(s.B, s.Lq, s.H, RA_BF16, s.c, s.N, r,
                                                           (ra_placement_t)place, 256);
        CHECK(k >= 1 && k <= 64);
      }
  }
  // Validation: each case fails on the host before any launch.
  const int before = ra::g_launches;
  float* const F = reinterpret_cast<float*>(P);
  CHECK(ra_blockwise_attn_fwd(P, P, P, nullptr, 1, 32, 32, 0, 0, 1, 64, 1, 128, RA_BF16, P, F,
                              nullptr) == RA_E_INVALID);                       // N = 0
  CHECK(ra_blockwise_attn_fwd(P, P, P, nullptr, 1, 48, 32, 4, 0, 1, 96, 1, 128, RA_BF16, P, F,
                              nullptr) == RA_E_UNSUPPORTED);                   // chunk % 32
  CHECK(ra_blockwise_attn_fwd(P, P, P, nullptr, 1, 32, 32, 4, 0, 1, 64, 1, 96, RA_BF16, P, F,
                              nullptr) == RA_E_UNSUPPORTED);                   // D = 96
  CHECK(ra_blockwise_attn_fwd(P + 2, P, P, nullptr, 1, 32, 32, 4, 0, 1, 64, 1, 128, RA_BF16, P,
                              F, nullptr) == RA_E_INVALID);                    // misaligned q
  CHECK(ra_blockwise_attn_fwd_split(P, P, P, nullptr, 1, 32, 32, 4, 0, RA_PLACE_STRIPED, 1, 64, 1,
                                    128, RA_BF16, P, F, nullptr, 0, nullptr, 0,
                                    nullptr) == RA_E_INVALID);                 // 0 splits
  CHECK(ra_blockwise_attn_bwd_split(P, P, P, nullptr, 1, 32, 32, 4, 0, RA_PLACE_CONTIGUOUS, 1, 64,
                                    1, 128, (ra_dtype_t)5, P, F, P, F, F, F, F, 1, nullptr, 0,
                                    nullptr) == RA_E_UNSUPPORTED);             // unknown dtype
  CHECK(ra_blockwise_attn_bwd_split(P, P, P, nullptr, 3, 32, 32, 4, 0, RA_PLACE_STRIPED, 1, 64,
                                    1, 128, RA_F32, P, F, P, F, F, F, F, 1, nullptr, 0,
                                    nullptr) == RA_E_UNSUPPORTED);             // striped c = 3
  CHECK(ra_blockwise_ffn(P, P, P, P, P, 1, 64, 64, 128, 48, RA_BF16, P, P, 1 << 20, nullptr) ==
        RA_E_INVALID);                                                        // chunk 48 of 64
  CHECK(std::strlen(ra_last_error()) > 0);
  CHECK(ra::g_launches == before);
  CHECK(ra_blockwise_ffn(P, P, P, P, P, 1, 64, 64, 128, 32, RA_BF16, P, P, 1 << 20, nullptr) ==
        RA_OK);
  CHECK(ra::g_launches == before + 1);

  // Decoding: the split grid the host derives covers every cache row, the
  // workspace split between numerators and carries, rejections launch
  // nothing.
  for (int64_t n_new : {1, 3, 8, 13, 256}) {
    for (int32_t S : {1, 5, 64, 1024}) {
      const int64_t B = 2, H = 32, D = 128, ci = 524287 - n_new;
      const int64_t ws = ra_attn_decode_workspace_bytes(B, n_new, H, D, S);
      const int n0 = ra::g_launches;
      CHECK(ra_attn_decode(P, P, P, ci, ci + n_new, B, n_new, H, D, RA_BF16, S,
                           S > 1 ? P : nullptr, ws, P, F, nullptr) == RA_OK);
      CHECK(ra::g_launches == n0 + 1);
      const ra::DecParams& d = ra::g_dec;
      CHECK(d.n_keys == ci + n_new);
      CHECK(d.split_keys % 64 == 0);
      CHECK((int64_t)d.key_splits * d.split_keys >= d.n_keys);
      CHECK((int64_t)d.q_groups * ra::g_dec_nq >= n_new);
      CHECK((int64_t)(d.q_groups - 1) * ra::g_dec_nq < n_new);
      if (S > 1) {
        CHECK(d.part_o == reinterpret_cast<float*>(P));
        CHECK(d.part_ml == d.part_o + (int64_t)S * B * H * n_new * D);
        CHECK(reinterpret_cast<const char*>(d.part_ml + 2LL * S * B * H * n_new) == P + ws);
      } else {
        CHECK(d.part_o == nullptr && d.part_ml == nullptr);
      }
    }
  }
  {
    const int n0 = ra::g_launches;
    CHECK(ra_attn_decode(P, P, P, 100, 100, 1, 1, 2, 128, RA_BF16, 1, nullptr, 0, P, F,
                         nullptr) == RA_E_INVALID);                          // row 100 missing
    CHECK(ra_attn_decode(P, P, P, 0, 300, 1, 257, 2, 128, RA_BF16, 1, nullptr, 0, P, F,
                         nullptr) == RA_E_UNSUPPORTED);                      // a prefill
    CHECK(ra_attn_decode(P, P, P, 10, 300, 1, 1, 2, 128, RA_BF16, 2, P, 100, P, F,
                         nullptr) == RA_E_INVALID);                          // short workspace
    CHECK(ra_attn_decode(P, P, P, 10, 300, 0, 1, 2, 128, RA_BF16, 2, nullptr, 0, nullptr,
                         nullptr, nullptr) == RA_OK);                        // empty batch
    CHECK(ra_attn_decode(P, P, P, INT64_MAX, 300, 1, 4, 2, 128, RA_BF16, 1, nullptr, 0, P, F,
                         nullptr) == RA_E_INVALID);                          // no wrap-around
    CHECK(ra_attn_decode(P, P, P, 0, INT64_MIN, 1, 4, 2, 128, RA_BF16, 1, nullptr, 0, P, F,
                         nullptr) == RA_E_INVALID);
    CHECK(ra::g_launches == n0);
  }
  CHECK(ra_attn_decode_key_splits(1, 1, 32, 524287, 256) == 64);
  CHECK(ra_attn_decode_key_splits(INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX, 256) == 1);
  CHECK(ra_attn_decode_key_splits(1LL << 30, 1, 1LL << 30, 1000, 256) == 1);
  CHECK(ra_attn_decode_key_splits(1, 1, 1, (1LL << 48) - 1, 1 << 30) == 1024);
  std::printf("%s: %d failure(s)\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
