// Host-side parts of the C ABI: error text, size queries and launch heuristics.
#include <algorithm>
#include <cstring>

#include "moe_internal.h"

namespace moe {

static thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return MOE_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace moe

using namespace moe;

extern "C" const char* moe_last_error(void) { return g_err; }

extern "C" int32_t moe_abi_version(void) { return 6; }

extern "C" int moe_align_capacity(int64_t M, int32_t top_k, int32_t n_local, int32_t block_m,
                                  int64_t* sorted_len, int64_t* blocks_len) {
  MOE_REQUIRE(sorted_len && blocks_len, MOE_EINVAL, "moe_align_capacity: null output pointer");
  MOE_REQUIRE(M >= 0 && top_k >= 1 && n_local >= 1 && block_m >= 1, MOE_EINVAL,
              "moe_align_capacity: M=%lld top_k=%d n_local=%d block_m=%d out of range",
              (long long)M, top_k, n_local, block_m);
  const int64_t numel = M * top_k;
  const int64_t worst = numel + std::min<int64_t>(n_local, numel) * (block_m - 1);
  const int64_t blocks = (worst + block_m - 1) / block_m;
  *sorted_len = blocks * block_m;
  *blocks_len = blocks;
  return ok();
}

extern "C" int moe_w4a16_prepared_size(moe_qtype q, int32_t E, int32_t N, int32_t K, uint32_t flags,
                                       int32_t has_bias, int32_t* N_out, int32_t* K_out,
                                       size_t* bytes) {
  MOE_REQUIRE(valid_qtype(q), MOE_EINVAL, "unknown qtype %d", (int)q);
  MOE_REQUIRE(E >= 1 && N >= 1 && K >= 1, MOE_EINVAL, "E=%d N=%d K=%d must be positive", E, N, K);
  MOE_REQUIRE((flags & ~(MOE_PREP_GATE_UP | MOE_PREP_INTERLEAVED | MOE_PREP_PAD | MOE_PREP_ACT_ORDER)) == 0,
              MOE_EINVAL, "unknown prepare flags 0x%x", flags);
  MOE_REQUIRE(!(flags & MOE_PREP_ACT_ORDER) || pair_grouped(q), MOE_EUNSUPPORTED,
              "MOE_PREP_ACT_ORDER (g_idx) is defined for the int4 formats only");
  MOE_REQUIRE(!(flags & MOE_PREP_ACT_ORDER) || (K % 128 == 0 && K <= kMaxActOrderK), MOE_EUNSUPPORTED,
              "MOE_PREP_ACT_ORDER: K=%d must be a multiple of 128 and at most %d", K, kMaxActOrderK);
  MOE_REQUIRE(!(flags & MOE_PREP_INTERLEAVED) || (flags & MOE_PREP_GATE_UP), MOE_EINVAL,
              "MOE_PREP_INTERLEAVED needs MOE_PREP_GATE_UP");
  const int g = group_of(q);
  MOE_REQUIRE(K % g == 0, MOE_EUNSUPPORTED, "K=%d is not a multiple of the group size %d", K, g);
  const bool pad = flags & MOE_PREP_PAD;
  int nout = N, kout = K;
  if (flags & MOE_PREP_GATE_UP) {
    MOE_REQUIRE(N % 2 == 0, MOE_EINVAL, "gate/up rows: N=%d must be even", N);
    const int I = N / 2;
    const int Ip = pad ? (I + kTileK - 1) / kTileK * kTileK : I;
    MOE_REQUIRE(Ip % kTileN == 0, MOE_EUNSUPPORTED,
                "gate/up halves of %d rows are not a multiple of %d (use MOE_PREP_PAD)", I, kTileN);
    nout = 2 * Ip;
  } else {
    MOE_REQUIRE(N % kTileN == 0, MOE_EUNSUPPORTED, "N=%d is not a multiple of %d", N, kTileN);
  }
  if (pad) kout = (K + kTileK - 1) / kTileK * kTileK;
  MOE_REQUIRE(kout % kTileK == 0, MOE_EUNSUPPORTED,
              "K=%d is not a multiple of %d (use MOE_PREP_PAD)", K, kTileK);
  if (pair_grouped(q))
    MOE_REQUIRE(kout % 128 == 0, MOE_EUNSUPPORTED, "int4: K=%d must be a multiple of 128", kout);
  const size_t tiles = (size_t)E * (nout / kTileN) * (kout / kTileK);
  size_t total = align256(tiles * kTileBytes);
  total += align256(tiles * (size_t)scale_bytes_per_tile(q));
  if (q == MOE_Q_NVFP4_G16) total += align256((size_t)E * 4);
  if (has_bias) total += align256((size_t)E * nout * 2);
  if (flags & MOE_PREP_ACT_ORDER) total += align256((size_t)E * K * 4);
  if (N_out) *N_out = nout;
  if (K_out) *K_out = kout;
  if (bytes) *bytes = total;
  return ok();
}

// BLOCK_SIZE_M for the align.  The Muse Spark experiment picks from (8, 16, 32, 48, 64) by the
// expected rows per expert; here the choice also selects the kernel: up to 16 rows per local
// expert (if every slot were local) go to the streaming decode kernel, larger counts to MFMA
// tiles of 32/64/128 rows.  Counting every slot (not only the expected local share) keeps skewed
// routing, where a few local experts take most slots, on the MFMA tiles that share weight reads.
// 128-row tiles halve the dequantisation per flop against 64-row ones but leave half as many
// workgroups; measured, they pay once an expert averages 256 rows and there are at least 8192
// slots (64 full blocks), below that the smaller grid and the padding cost more.
// Within the decode range the kernel is chosen by moe_gemm_choose (16-slot blocks run either the
// streaming kernel or the MFMA kernel); only a short K (<= 1024, int4 here) beyond the fused-align
// range (> 64 slots) with about 32 or more live slots takes 32-slot MFMA blocks (measured, whole
// int4 layer: 22.6 us streaming against 25.5 us MFMA at 64 slots, tie at 96, 27.8 against 25.7 at
// 128; the streaming kernel there also takes the align fused in).
extern "C" int moe_choose_block_m(int64_t numel, int32_t n_local, int64_t expected_live, int32_t K,
                                  int32_t* block_m) {
  MOE_REQUIRE(block_m && numel >= 0 && n_local >= 1, MOE_EINVAL, "moe_choose_block_m: bad arguments");
  const double rows = (double)numel / n_local;
  const int64_t live = expected_live > 0 ? std::min(expected_live, numel) : numel;
  int b = 16;
  if (rows > 16) b = 32;
  if (rows > 48) b = 64;
  // 128-slot blocks from 8192 slots once an expert averages 256 rows, or once the slots expected
  // live average 48 per expert: then most experts fit one 128-slot block, whose unused 16-slot
  // groups the MFMA kernel skips, and each expert's weights are dequantised once instead of in
  // two 64-slot blocks (measured: MXFP4 M=2048, 64 live rows per expert, 591 us against 623 us;
  // the NVFP4 slice at M=256, 8 expected live rows per expert, keeps 64: 328 against 387 us)
  if (numel >= 8192 && (rows >= 256 || (double)live / n_local >= 48)) b = 128;
  if (b == 16 && live >= 32 && K > 0 && K <= 1024 && numel > 64) b = 32;
  *block_m = b;
  return ok();
}

namespace moe {
// The streaming decode kernel over min(numel, E) live blocks.  Measured (cold weights, NVFP4 and
// MXFP4 slices): four 16-row tiles per wave once about 8 blocks are live, else two; then the
// smallest K split that gives at least 24 waves per CU.  The one-column MFMA streams faster than
// the dot-product path (gemv_rows > 0), which stays available.
moe_gemm_config stream_config(const moe_weights* W, int64_t numel, int num_cus) {
  moe_gemm_config c{};
  c.kernel = MOE_GEMM_DECODE;
  c.gemv_rows = 0;
  const int64_t nt = W->N / kTileN;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(numel, W->n_experts));
  c.ng = blocks >= 8 ? 4 : 2;
  const int64_t items = blocks * ((nt + c.ng - 1) / c.ng);
  c.ksplit = 1;
  while (c.ksplit < 8 && items * c.ksplit < 24ll * (num_cus > 0 ? num_cus : 256)) c.ksplit *= 2;
  return c;
}
}  // namespace moe

extern "C" int moe_gemm_choose_occ(const moe_weights* W, int64_t numel, int32_t block_m, int32_t num_cus,
                                   const int32_t resident[3], moe_gemm_config* cfg) {
  MOE_REQUIRE(W && cfg && resident, MOE_EINVAL, "moe_gemm_choose: null pointer");
  MOE_REQUIRE(block_m >= 1 && numel >= 0, MOE_EINVAL, "moe_gemm_choose: bad block_m/numel");
  if (num_cus <= 0) num_cus = 256;
  moe_gemm_config c{};
  const int nt = W->N / kTileN;
  if (block_m <= 16 && W->K >= 2048 && numel >= 32) {
    // 16-slot blocks with about 32 or more live slots of long-K weights: the MFMA kernel (its
    // global->LDS stream, two tiles per wave) outruns the streaming kernel.  Measured, whole
    // layers: NVFP4 slice with 32 / 64 live slots 153.5 -> 130.9 / 160.0 -> 145.8 us, MXFP4 with
    // 128 live 255 -> 210 us (32-slot MFMA blocks: 149 / 160 / 218 us; four tiles per wave 146 /
    // 157 / 227 us); with 16 live slots the streaming kernel still wins (94 against 107 us).
    c.kernel = MOE_GEMM_MFMA;
    c.ng = 2;
    c.group_m = default_group_m(W->K, block_m);
  } else if (block_m <= 16) {
    c = stream_config(W, numel, num_cus);
  } else {
    // prefill.  Two 16-row tiles per wave by default.  Four (the dequantised weights then feed
    // twice the MFMAs per load of the block's activations) when the weights stream from HBM
    // through long K loops (64-slot blocks and K >= 2048) or the blocks hold 128 slots, and the
    // four-tile grid needs no more rounds of resident workgroups than the two-tile one -- the
    // residency per CU of each variant is the kernel's own (registers and LDS, from the
    // occupancy API: 2 for the 128-slot four-tile kernels, 4 for the 64-slot ones).  One tile
    // when two would not give every CU a workgroup.  Measured on the int4, NVFP4 and MXFP4
    // prefill shapes: MXFP4 M=2048 gate/up 565 -> 428 us and down 291 -> 242 us, NVFP4 M=256
    // down 163 -> 141 us and gate/up 271 -> 232 us, NVFP4 M=1024 (64-row blocks) gate/up
    // 583 -> 507 us with four tiles; the int4 GEMMs (K <= 1024, 64-slot blocks) are faster with
    // two, and the int4 down GEMM at M = 2304 (320 workgroups with two tiles) 16.3 us against
    // 18.2 us with one tile and twice the workgroups.
    c.kernel = MOE_GEMM_MFMA;
    const int64_t mblocks = numel / block_m + std::min<int64_t>(numel, W->n_experts);
    const bool streamed = block_m >= 64 && W->K >= 2048;
    auto grid = [&](int ng) { return (int64_t)((nt + 4 * ng - 1) / (4 * ng)) * mblocks; };
    auto rounds = [&](int ng, int res) {
      const int64_t slots = (int64_t)std::max(1, res) * num_cus;
      return (grid(ng) + slots - 1) / slots;
    };
    c.ng = 2;
    if ((block_m >= 128 || streamed) && grid(4) >= num_cus && rounds(4, resident[2]) <= rounds(2, resident[1]))
      c.ng = 4;
    if (grid(2) < num_cus) c.ng = 1;
    c.group_m = default_group_m(W->K, block_m);
  }
  *cfg = c;
  return ok();
}

extern "C" int moe_gemm_choose(const moe_weights* W, int64_t numel, int32_t block_m, int32_t num_cus,
                               moe_gemm_config* cfg) {
  MOE_REQUIRE(W && cfg, MOE_EINVAL, "moe_gemm_choose: null pointer");
  // the MFMA kernels' residency on this device; without one, the two workgroups per CU their
  // launch bound guarantees
  int32_t resident[3] = {2, 2, 2};
  if (block_m == 32 || block_m == 64 || block_m == 128) {
    int32_t r[3];
    if (moe_gemm_occupancy(W, block_m, (W->flags & MOE_PREP_GATE_UP) != 0, r) == MOE_OK)
      for (int j = 0; j < 3; ++j) resident[j] = r[j];
  }
  return moe_gemm_choose_occ(W, numel, block_m, num_cus, resident, cfg);
}
