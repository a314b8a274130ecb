// Host-side checks of libmoe_w4a16 under AddressSanitizer and UndefinedBehaviorSanitizer: the
// size queries, the launch heuristics and every validation path that returns before a launch
// (device pointers here are fake addresses that are never dereferenced, so no kernel runs and no
// GPU is needed).  Built and run by tests/test_host_sanitizers.py; prints "ok" when every check
// holds, exits non-zero on the first failure.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include <vector>

#include "moe_w4a16.h"
#include "moe_internal.h"

namespace moe {
int device_cu_count() { return 256; }  // (the GEMM sources that define it are not linked here)
}
// (the GEMM sources are not linked: no device answers, so moe_gemm_choose takes the launch bound)
extern "C" int moe_gemm_occupancy(const moe_weights*, int32_t, int32_t, int32_t*) { return MOE_EHIP; }

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, moe_last_error()); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
  // ---- align capacity: numel + min(E, numel) (B - 1), rounded up to whole blocks
  const int64_t cases[][4] = {{0, 8, 32, 16}, {1, 8, 32, 16}, {123, 2, 8, 32}, {4096, 8, 32, 128},
                              {2048, 4, 128, 64}, {5, 3, 512, 256}, {1, 1, 1, 1}, {1 << 20, 8, 256, 16}};
  for (const auto& c : cases) {
    int64_t s = -1, b = -1;
    CHECK(moe_align_capacity(c[0], (int32_t)c[1], (int32_t)c[2], (int32_t)c[3], &s, &b) == MOE_OK);
    const int64_t numel = c[0] * c[1], worst = numel + (c[2] < numel ? c[2] : numel) * (c[3] - 1);
    CHECK(b == (worst + c[3] - 1) / c[3] && s == b * c[3]);
  }
  int64_t s = 0, b = 0;
  CHECK(moe_align_capacity(-1, 8, 32, 16, &s, &b) == MOE_EINVAL);
  CHECK(moe_align_capacity(1, 8, 32, 0, &s, &b) == MOE_EINVAL);
  CHECK(moe_align_capacity(1, 8, 32, 16, nullptr, &b) == MOE_EINVAL);
  CHECK(std::strlen(moe_last_error()) > 0);

  // ---- prepared sizes: every format and flag combination, valid and invalid
  const moe_qtype qs[] = {MOE_Q_INT4_G128, MOE_Q_NVFP4_G16, MOE_Q_MXFP4_G32, MOE_Q_INT4ZP_G128, MOE_Q_INT4ZPF_G128};
  for (moe_qtype q : qs) {
    for (uint32_t flags = 0; flags < 16; ++flags) {
      for (int K : {128, 192, 2880, 4096}) {
        int32_t n = 0, k = 0;
        size_t bytes = 0, bytes_bias = 0;
        const int rc = moe_w4a16_prepared_size(q, 4, 5760, K, flags, 0, &n, &k, &bytes);
        if (rc == MOE_OK) {
          CHECK(moe_w4a16_prepared_size(q, 4, 5760, K, flags, 1, &n, &k, &bytes_bias) == MOE_OK);
          CHECK(bytes_bias > bytes && bytes % 256 == 0 && k >= K && k % 64 == 0 && n % 16 == 0);
          const bool ao = flags & MOE_PREP_ACT_ORDER;
          CHECK(!ao || (q == MOE_Q_INT4_G128 || q == MOE_Q_INT4ZP_G128 || q == MOE_Q_INT4ZPF_G128));
          if (ao) {
            size_t plain = 0;
            CHECK(moe_w4a16_prepared_size(q, 4, 5760, K, flags & ~MOE_PREP_ACT_ORDER, 0, &n, &k, &plain) == MOE_OK);
            CHECK(bytes - plain == (size_t)4 * K * 4);
          }
        } else {
          CHECK(rc == MOE_EINVAL || rc == MOE_EUNSUPPORTED);
        }
      }
    }
  }
  int32_t n = 0, k = 0;
  size_t bytes = 0;
  CHECK(moe_w4a16_prepared_size((moe_qtype)9, 4, 64, 256, 0, 0, &n, &k, &bytes) == MOE_EINVAL);
  CHECK(moe_w4a16_prepared_size(MOE_Q_INT4_G128, 4, 64, 256, 0x10, 0, &n, &k, &bytes) == MOE_EINVAL);
  CHECK(moe_w4a16_prepared_size(MOE_Q_INT4_G128, 4, 64, 32768, MOE_PREP_ACT_ORDER, 0, &n, &k, &bytes) ==
        MOE_EUNSUPPORTED);

  // ---- prepare: argument checks before any launch
  moe_weights d{};
  void* out = fake(1 << 20);
  const uint8_t* c8 = static_cast<const uint8_t*>(fake(1 << 16));
  const int32_t* g32 = static_cast<const int32_t*>(fake(1 << 16));
  CHECK(moe_w4a16_prepare(MOE_Q_INT4ZP_G128, c8, c8, nullptr, nullptr, nullptr, nullptr, 4, 64, 256, 0, out,
                          1 << 20, &d, nullptr) == MOE_EINVAL);                       // no zero points
  CHECK(moe_w4a16_prepare(MOE_Q_INT4_G128, c8, c8, nullptr, nullptr, nullptr, nullptr, 4, 64, 256,
                          MOE_PREP_ACT_ORDER, out, 1 << 20, &d, nullptr) == MOE_EINVAL);  // flag, no g_idx
  CHECK(moe_w4a16_prepare(MOE_Q_INT4_G128, c8, c8, nullptr, nullptr, nullptr, g32, 4, 64, 256, 0, out,
                          1 << 20, &d, nullptr) == MOE_EINVAL);                       // g_idx, no flag
  CHECK(moe_w4a16_prepare(MOE_Q_NVFP4_G16, c8, c8, nullptr, nullptr, nullptr, nullptr, 4, 64, 256, 0, out,
                          1 << 20, &d, nullptr) == MOE_EINVAL);                       // no global scale
  CHECK(moe_w4a16_prepare(MOE_Q_INT4_G128, c8, c8, nullptr, nullptr, nullptr, nullptr, 4, 64, 256, 0, out,
                          16, &d, nullptr) == MOE_ESIZE);                             // out too small
  CHECK(moe_w4a16_prepare(MOE_Q_INT4_G128, c8, c8, nullptr, nullptr, nullptr, nullptr, 4, 64, 256, 0,
                          fake((1 << 20) + 8), 1 << 20, &d, nullptr) == MOE_EINVAL);  // misaligned out

  // ---- heuristics
  int32_t bm = 0, prev = 0;
  for (int64_t numel = 0; numel <= (1 << 18); numel = numel ? numel * 2 : 1) {
    CHECK(moe_choose_block_m(numel, 32, numel / 4, 4096, &bm) == MOE_OK);
    CHECK(bm == 16 || bm == 32 || bm == 64 || bm == 128);
    CHECK(bm >= prev);
    prev = bm;
  }
  moe_weights w{};
  w.qtype = MOE_Q_NVFP4_G16;
  w.n_experts = 32;
  w.N = 8192;
  w.K = 4096;
  w.flags = MOE_PREP_GATE_UP;
  moe_gemm_config cfg{};
  for (int64_t numel : {1, 8, 64, 512, 4096, 32768}) {
    for (int32_t block : {16, 64, 128}) {
      CHECK(moe_gemm_choose(&w, numel, block, 256, &cfg) == MOE_OK);
      CHECK(cfg.ng == 1 || cfg.ng == 2 || cfg.ng == 4);
      // 16-slot blocks: the streaming kernel, or the MFMA kernel from 32 live slots of long-K weights
      const bool stream = block <= 16 && numel < 32;
      CHECK(!stream || (cfg.kernel == MOE_GEMM_DECODE && cfg.ksplit >= 1 && cfg.ksplit <= 8));
      CHECK(stream || (cfg.kernel == MOE_GEMM_MFMA && cfg.group_m >= 1 && cfg.group_m <= 8));
    }
  }
  CHECK(moe_gemm_choose(nullptr, 8, 16, 256, &cfg) == MOE_EINVAL);
  // with any residency the prefill choice is one of the built tile counts
  for (int r4 : {1, 2, 3, 4, 8})
    for (int64_t numel : {256, 2048, 23283, 1 << 20})
      for (int32_t block : {32, 64, 128}) {
        const int32_t res[3] = {8, 4, r4};
        CHECK(moe_gemm_choose_occ(&w, numel, block, 256, res, &cfg) == MOE_OK);
        CHECK(cfg.kernel == MOE_GEMM_MFMA && (cfg.ng == 1 || cfg.ng == 2 || cfg.ng == 4));
      }
  CHECK(moe_gemm_choose_occ(&w, 8, 64, 256, nullptr, &cfg) == MOE_EINVAL);

  moe_requant_config rq{};
  for (int32_t E : {1, 8, 32, 256, 1024})
    for (int32_t max_m : {0, 1, 8, 512})
      for (int32_t K : {128, 1040, 7168})
        for (int32_t expected : {0, 1, 33, 1 << 20}) {
          CHECK(moe_fp8_requant_choose(E, max_m, K, expected, 256, &rq) == MOE_OK);
          CHECK(rq.workgroups >= 1 && rq.workgroups <= 2048 && (rq.unroll == 1 || rq.unroll == 2 || rq.unroll == 4));
        }
  CHECK(moe_fp8_requant_choose(8, 8, 7168, 0, 0, &rq) == MOE_EINVAL);

  // ---- requant and act-order gather: every rejection happens before a launch
  const uint8_t* x8 = static_cast<const uint8_t*>(fake(1 << 24));
  const float* f32 = static_cast<const float*>(fake(1 << 16));
  uint8_t* o8 = static_cast<uint8_t*>(fake(1 << 26));
  moe_requant_config bad{0, 1};
  CHECK(moe_fp8_requant(x8, f32, 16, 2, 1, g32, f32, 8, 8, 256, 128, o8, &bad, nullptr) == MOE_EINVAL);
  CHECK(moe_fp8_requant(x8, f32, 16, 2, 1, g32, f32, 8, 8, 256, 8, o8, nullptr, nullptr) == MOE_EUNSUPPORTED);
  CHECK(moe_fp8_requant(x8, f32, 16, 2, 1, g32, f32, 2000, 8, 256, 128, o8, nullptr, nullptr) ==
        MOE_EUNSUPPORTED);
  CHECK(moe_fp8_requant(x8, f32, 16, 2, 1, g32, f32, 8, 8, 200, 128, o8, nullptr, nullptr) == MOE_EINVAL);
  CHECK(moe_fp8_requant(x8, f32, 16, 2, 1, g32, f32, 8, 8, 256, 128, const_cast<uint8_t*>(x8) + 64, nullptr,
                        nullptr) == MOE_EINVAL);                                      // partial overlap
  CHECK(moe_fp8_requant(nullptr, nullptr, 0, 0, 0, nullptr, nullptr, 0, 8, 256, 128, nullptr, nullptr,
                        nullptr) == MOE_OK);                                          // E = 0: no launch
  const uint16_t* s16 = static_cast<const uint16_t*>(fake(1 << 16));
  uint16_t* d16 = static_cast<uint16_t*>(fake(1 << 20));
  CHECK(moe_permute_cols(s16, 256, 2, g32, 252, 4, g32, 8, d16, 256, nullptr) == MOE_EINVAL);
  CHECK(moe_permute_cols(s16, 128, 2, g32, 256, 4, g32, 8, d16, 256, nullptr) == MOE_EINVAL);
  CHECK(moe_permute_cols(s16, 256, 0, g32, 256, 4, g32, 8, d16, 256, nullptr) == MOE_EINVAL);
  CHECK(moe_permute_cols(s16, 256, 2, g32, 256, 4, g32, 8, d16 + 1, 256, nullptr) == MOE_EINVAL);
  CHECK(moe_permute_cols(nullptr, 256, 2, nullptr, 256, 4, nullptr, 0, nullptr, 256, nullptr) == MOE_OK);

  // ---- the MFMA GEMM's XCD-aware launch order: a bijection from launch index to (align block,
  // column block) on every grid it is launched with (nblk column blocks x any number of align
  // blocks, any group size), including grids whose last round of groups is partial
  for (int nblk : {1, 2, 3, 5, 8, 16, 32, 33})
    for (int blocks = 1; blocks <= 97; blocks += (blocks < 20 ? 1 : 7))
      for (int gm : {1, 2, 3, 4, 8, 16}) {
        const int G = nblk * blocks;
        std::vector<char> seen((size_t)G, 0);
        bool in_range = true, once = true;
        for (int P = 0; P < G; ++P) {
          int mb = -1, nb = -1;
          moe::xcd_grouped_block(G, P, nblk, gm, mb, nb);
          if (mb < 0 || mb >= blocks || nb < 0 || nb >= nblk) { in_range = false; break; }
          char& v = seen[(size_t)mb * nblk + nb];
          if (v) once = false;
          v = 1;
        }
        CHECK(in_range && once);
      }
  // whole groups of gm blocks go to one XCD (launch index mod 8) while full rounds last
  {
    const int nblk = 4, blocks = 64, gm = 2, G = nblk * blocks;
    bool same_xcd = true;
    for (int P = 0; P < G; ++P)
      for (int Q = 0; Q < G; ++Q) {
        int mb1, nb1, mb2, nb2;
        moe::xcd_grouped_block(G, P, nblk, gm, mb1, nb1);
        moe::xcd_grouped_block(G, Q, nblk, gm, mb2, nb2);
        if (mb1 / gm == mb2 / gm && P % 8 != Q % 8) same_xcd = false;
      }
    CHECK(same_xcd);
  }

  CHECK(moe_abi_version() == 6);
  if (failures) {
    std::printf("%d checks failed\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
