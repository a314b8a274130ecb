// moe_w4a16_gemm: argument validation, launch-configuration choice and dispatch to the
// streaming decode kernel (moe_gemm_stream.h), the dot-product decode kernel (moe_gemm_decode.h)
// or the MFMA kernel (moe_gemm_mfma.h), instantiated per format in moe_gemm_{int4,int4zp,nvfp4,
// mxfp4}.hip and moe_gemm_stream_*.hip.
//
// The computation is that of moe_wna16_marlin_gemm in the Muse Spark experiment and of the
// Marlin template in the "sglang PR 31552" summary: for each block of sorted slots of one
// expert, C[slot] = dequant(W[e]) . A[slot / top_k] with fp32 accumulation, the per-expert bias
// added at the end (kHasBias there, a template parameter here) and bf16 results.
#include <mutex>

#include "moe_gemm_common.h"

namespace moe {

int device_cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static bool al(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

// Residency of the MFMA kernel variants, per device: the occupancy API is asked once per
// (device, format, bias, gated, block_m) and the answer kept.
struct ResidencyKey {
  int dev, qtype, bias, gated, block_m;
  bool operator==(const ResidencyKey& o) const {
    return dev == o.dev && qtype == o.qtype && bias == o.bias && gated == o.gated && block_m == o.block_m;
  }
};
static std::mutex g_res_mu;
static ResidencyKey g_res_key[256];
static int g_res_val[256][3];
static int g_res_n;


// Routed mode (topk_ids set): the align of the numel <= kFusedAlignSlots slots is computed inside
// the streaming kernel, and sorted_token_ids / expert_ids / num_tokens_post_padded / slot_local
// are its outputs instead of inputs.
// Fused weighted sum (moe_w4a16_gemm_combine): the combine's inputs and output.
struct CombineSpec {
  const float* gw;
  const int32_t* live;
  uint16_t* out;
  int64_t ldo;
  int32_t* cnt;
  int64_t cnt_len;
  int32_t k;
  int64_t M;
  float rsf;
  bool clear;   // zero the first M * strips counters right before the GEMM launch
};

// ---------------------------------------------------------------------------- library scratch
// Arrival counters of moe_w4a16_gemm_combine_noalloc, for callers that cannot allocate: one
// array per device, in the library's own device memory, held until the process ends.  Host code
// never uses the array's name as an address (on the host it is only a stand-in): its device
// address is looked up once per device with hipGetSymbolAddress and kept in g_scratch_ptr.
static __device__ __align__(256) int32_t scratch[kNoAllocCounters];
static std::mutex g_scratch_mu;
static int32_t* g_scratch_ptr[64];

// The current device's copy of `scratch` (looked up on the first call on each device).
static int scratch_counters(int32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_EHIP, "moe_w4a16_gemm_combine_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  MOE_REQUIRE(dev >= 0 && dev < 64, MOE_EUNSUPPORTED, "moe_w4a16_gemm_combine_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_EHIP, "moe_w4a16_gemm_combine_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// A plain fill kernel (no memset node, so the clear may be captured in a HIP graph).
__global__ void zero_counters_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

static int zero_counters(int32_t* p, int64_t n, hipStream_t st) {
  if (n <= 0) return ok();
  const int64_t blocks = std::min<int64_t>(256, (n + 255) / 256);
  hipLaunchKernelGGL(zero_counters_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return check_launch("moe_w4a16_gemm_combine_noalloc (counter clear)");
}

static int gemm_impl(int act, float alpha, float limit, const uint16_t* A, int64_t a_rows, int32_t lda,
                     uint16_t* C, int32_t ldc, const moe_weights* W, const int32_t* sorted_token_ids,
                     const int32_t* expert_ids, const int32_t* num_tokens_post_padded, int64_t numel,
                     int32_t top_k, int32_t block_m, const moe_gemm_config* cfg, hipStream_t stream,
                     const int32_t* topk_ids = nullptr, int32_t expert_start = 0, int32_t* slot_local = nullptr,
                     const CombineSpec* cmb = nullptr) {
  MOE_REQUIRE(W, MOE_EINVAL, "moe_w4a16_gemm: null weights");
  MOE_REQUIRE(valid_qtype(W->qtype), MOE_EINVAL, "moe_w4a16_gemm: bad qtype %d", W->qtype);
  MOE_REQUIRE(W->n_experts >= 1 && W->N >= kTileN && W->N % kTileN == 0 && W->K >= kTileK &&
                  W->K % kTileK == 0,
              MOE_EINVAL, "moe_w4a16_gemm: weights E=%d N=%d K=%d not in the prepared layout",
              W->n_experts, W->N, W->K);
  MOE_REQUIRE(W->codes && W->scales, MOE_EINVAL, "moe_w4a16_gemm: weights without codes/scales");
  MOE_REQUIRE(W->qtype != MOE_Q_NVFP4_G16 || W->global_scale, MOE_EINVAL,
              "moe_w4a16_gemm: NVFP4 weights without global scales");
  const bool paired = act_paired(act);
  const int ncols = paired ? W->N / 2 : W->N;  // output columns
  if (paired)
    MOE_REQUIRE((W->flags & MOE_PREP_GATE_UP) && W->N % (2 * kTileN) == 0, MOE_EINVAL,
                "moe_w4a16_gemm_act: a gated activation needs a gate/up pair (prepared with MOE_PREP_GATE_UP)");
  if (act == kActRelu2)
    MOE_REQUIRE(!(W->flags & MOE_PREP_GATE_UP), MOE_EINVAL,
                "moe_w4a16_gemm_act: relu2 is non-gated: weights must not be a gate/up pair");
  MOE_REQUIRE(numel >= 0 && numel < (1 << 30), MOE_EUNSUPPORTED, "moe_w4a16_gemm: numel=%lld", (long long)numel);
  MOE_REQUIRE(top_k >= 1 && block_m >= 1, MOE_EINVAL, "moe_w4a16_gemm: top_k=%d block_m=%d", top_k, block_m);
  MOE_REQUIRE(a_rows >= (numel + top_k - 1) / top_k, MOE_EINVAL,
              "moe_w4a16_gemm: A has %lld rows, slots need %lld", (long long)a_rows,
              (long long)((numel + top_k - 1) / top_k));
  MOE_REQUIRE(lda >= W->K && lda % 8 == 0 && ldc >= ncols && ldc % 4 == 0, MOE_EINVAL,
              "moe_w4a16_gemm: lda=%d (>= K=%d, multiple of 8) ldc=%d (>= %d columns, multiple of 4)", lda,
              W->K, ldc, ncols);
  if (numel == 0) return ok();
  MOE_REQUIRE(A && C && sorted_token_ids && expert_ids && num_tokens_post_padded, MOE_EINVAL,
              "moe_w4a16_gemm: null pointer");
  MOE_REQUIRE(al(A, 16) && al(C, 8) && al(W->codes, 16) && al(W->scales, 4) && (!W->bias || al(W->bias, 8)),
              MOE_EUNSUPPORTED, "moe_w4a16_gemm: misaligned pointer (A 16 B, C 8 B, bias 8 B)");
  const int cus = device_cu_count();
  moe_gemm_config c{};
  if (cfg && cfg->kernel != MOE_GEMM_AUTO) {
    c = *cfg;
  } else {
    int rc = moe_gemm_choose(W, numel, block_m, cus, &c);
    if (rc) return rc;
    if (paired && c.ng < 2) c.ng = 2;  // the fused gated epilogue needs gate/up tile pairs
  }
  MOE_REQUIRE(!paired || c.ng == 2 || c.ng == 4, MOE_EINVAL,
              "moe_w4a16_gemm_act: a fused gated activation needs ng 2 or 4 (gate/up tile pairs), got %d", c.ng);
  if (topk_ids) {
    MOE_REQUIRE(c.kernel == MOE_GEMM_DECODE && c.gemv_rows == 0, MOE_EUNSUPPORTED,
                "moe_w4a16_gemm_act_routed: the fused align runs in the streaming decode kernel "
                "(kernel DECODE, gemv_rows 0)");
    MOE_REQUIRE(slot_local, MOE_EINVAL, "moe_w4a16_gemm_act_routed: null slot_local_ids");
  }
  int64_t cap = 0, cap_blocks = 0;
  int rc = moe_align_capacity(numel, 1, W->n_experts, block_m, &cap, &cap_blocks);
  if (rc) return rc;
  GemmArgs a{A, lda, C, ldc,
             static_cast<const uint8_t*>(W->codes), static_cast<const uint8_t*>(W->scales),
             W->global_scale, W->bias, sorted_token_ids, expert_ids, num_tokens_post_padded,
             (int32_t)numel, top_k, block_m, W->N, W->K, W->n_experts, alpha, limit, c.group_m,
             topk_ids, expert_start, (int32_t)cap, (int32_t)cap_blocks, const_cast<int32_t*>(sorted_token_ids),
             const_cast<int32_t*>(expert_ids), const_cast<int32_t*>(num_tokens_post_padded), slot_local};
  const bool bias = W->bias != nullptr;
  if (cmb) {
    MOE_REQUIRE(c.kernel == MOE_GEMM_DECODE && c.gemv_rows == 0, MOE_EUNSUPPORTED,
                "moe_w4a16_gemm_combine: the fused weighted sum runs in the streaming decode kernel "
                "(block_m <= 16; kernel DECODE, gemv_rows 0)");
    MOE_REQUIRE(c.ng == 1 || c.ng == 2 || c.ng == 4, MOE_EINVAL, "moe_w4a16_gemm_combine: ng=%d", c.ng);
    const int64_t strips = (W->N / kTileN + c.ng - 1) / c.ng;
    MOE_REQUIRE(cmb->cnt_len >= cmb->M * strips, MOE_ESIZE,
                "moe_w4a16_gemm_combine: %lld counters, need %lld", (long long)cmb->cnt_len,
                (long long)(cmb->M * strips));
    a.cmb_gw = cmb->gw;
    a.cmb_live = cmb->live;
    a.cmb_out = cmb->out;
    a.cmb_cnt = cmb->cnt;
    a.cmb_k = cmb->k;
    a.cmb_ntok = (int32_t)cmb->M;
    a.cmb_ldo = cmb->ldo;
    a.cmb_rsf = cmb->rsf;
  }
  if (c.kernel == MOE_GEMM_DECODE) {
    MOE_REQUIRE(block_m <= 16, MOE_EUNSUPPORTED, "moe_w4a16_gemm: decode kernel needs block_m <= 16");
    MOE_REQUIRE(c.ksplit >= 1 && c.ksplit <= 8, MOE_EINVAL, "moe_w4a16_gemm: decode ksplit=%d (1..8)", c.ksplit);
    MOE_REQUIRE(c.gemv_rows >= 0 && c.gemv_rows <= 4, MOE_EINVAL, "moe_w4a16_gemm: gemv_rows=%d (0..4)",
                c.gemv_rows);
    MOE_REQUIRE((int64_t)c.gemv_rows * W->K * 2 <= 32768, MOE_EUNSUPPORTED,
                "moe_w4a16_gemm: gemv_rows=%d x K=%d exceeds the 32 KiB activation stage", c.gemv_rows, W->K);
    if (c.gemv_rows == 0) {  // one-column MFMA on every block: the streaming kernel
      if (cmb && cmb->clear) {  // (every argument has been checked: the launches follow)
        const int64_t strips = (W->N / kTileN + c.ng - 1) / c.ng;
        int rcz = zero_counters(cmb->cnt, cmb->M * strips, stream);
        if (rcz) return rcz;
      }
      switch (W->qtype) {
        case MOE_Q_INT4_G128: return launch_gemm_stream<MOE_Q_INT4_G128>(bias, act, a, c, (int)cap_blocks, cus, stream);
        case MOE_Q_NVFP4_G16: return launch_gemm_stream<MOE_Q_NVFP4_G16>(bias, act, a, c, (int)cap_blocks, cus, stream);
        case MOE_Q_INT4ZP_G128: return launch_gemm_stream<MOE_Q_INT4ZP_G128>(bias, act, a, c, (int)cap_blocks, cus, stream);
        case MOE_Q_INT4ZPF_G128: return launch_gemm_stream<MOE_Q_INT4ZPF_G128>(bias, act, a, c, (int)cap_blocks, cus, stream);
        default: return launch_gemm_stream<MOE_Q_MXFP4_G32>(bias, act, a, c, (int)cap_blocks, cus, stream);
      }
    }
    switch (W->qtype) {
      case MOE_Q_INT4_G128: return launch_gemm_decode<MOE_Q_INT4_G128>(bias, act, a, c, (int)cap_blocks, cus, stream);
      case MOE_Q_NVFP4_G16: return launch_gemm_decode<MOE_Q_NVFP4_G16>(bias, act, a, c, (int)cap_blocks, cus, stream);
      case MOE_Q_INT4ZP_G128: return launch_gemm_decode<MOE_Q_INT4ZP_G128>(bias, act, a, c, (int)cap_blocks, cus, stream);
      case MOE_Q_INT4ZPF_G128: return launch_gemm_decode<MOE_Q_INT4ZPF_G128>(bias, act, a, c, (int)cap_blocks, cus, stream);
      default: return launch_gemm_decode<MOE_Q_MXFP4_G32>(bias, act, a, c, (int)cap_blocks, cus, stream);
    }
  }
  MOE_REQUIRE(c.kernel == MOE_GEMM_MFMA, MOE_EINVAL, "moe_w4a16_gemm: unknown kernel %d", c.kernel);
  MOE_REQUIRE(a_rows * (int64_t)lda * 2 <= (int64_t)UINT32_MAX, MOE_EUNSUPPORTED,
              "moe_w4a16_gemm: MFMA kernel addresses A with 32-bit byte offsets; A spans %lld bytes",
              (long long)(a_rows * (int64_t)lda * 2));
  MOE_REQUIRE(c.ng == 1 || c.ng == 2 || c.ng == 4, MOE_EINVAL, "moe_w4a16_gemm: ng=%d (1, 2 or 4)", c.ng);
  MOE_REQUIRE(c.group_m >= 0 && c.group_m <= 64, MOE_EINVAL, "moe_w4a16_gemm: group_m=%d (0..64)", c.group_m);
  if (c.group_m == 0) c.group_m = moe::default_group_m(W->K, block_m);
  a.group_m = c.group_m;
  a.border = c.block_order;
  MOE_REQUIRE((int64_t)((W->N / kTileN + 4 * c.ng - 1) / (4 * c.ng)) * cap_blocks < (1ll << 31),
              MOE_EUNSUPPORTED, "moe_w4a16_gemm: grid too large");
  switch (W->qtype) {
    case MOE_Q_INT4_G128: return launch_gemm_mfma<MOE_Q_INT4_G128>(bias, act, a, c, (int)cap_blocks, stream);
    case MOE_Q_NVFP4_G16: return launch_gemm_mfma<MOE_Q_NVFP4_G16>(bias, act, a, c, (int)cap_blocks, stream);
    case MOE_Q_INT4ZP_G128: return launch_gemm_mfma<MOE_Q_INT4ZP_G128>(bias, act, a, c, (int)cap_blocks, stream);
    case MOE_Q_INT4ZPF_G128: return launch_gemm_mfma<MOE_Q_INT4ZPF_G128>(bias, act, a, c, (int)cap_blocks, stream);
    default: return launch_gemm_mfma<MOE_Q_MXFP4_G32>(bias, act, a, c, (int)cap_blocks, stream);
  }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_gemm_occupancy(const moe_weights* W, int32_t block_m, int32_t gated, int32_t resident[3]) {
  MOE_REQUIRE(W && resident, MOE_EINVAL, "moe_gemm_occupancy: null pointer");
  MOE_REQUIRE(valid_qtype(W->qtype), MOE_EINVAL, "moe_gemm_occupancy: bad qtype %d", W->qtype);
  MOE_REQUIRE(block_m == 16 || block_m == 32 || block_m == 64 || block_m == 128, MOE_EINVAL,
              "moe_gemm_occupancy: block_m=%d (16, 32, 64 or 128)", block_m);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_EHIP, "moe_gemm_occupancy: hipGetDevice: %s", hipGetErrorString(e));
  }
  const ResidencyKey key{dev, W->qtype, W->bias != nullptr, gated != 0, block_m};
  std::lock_guard<std::mutex> lock(g_res_mu);
  for (int i = 0; i < g_res_n; ++i)
    if (g_res_key[i] == key) {
      for (int j = 0; j < 3; ++j) resident[j] = g_res_val[i][j];
      return ok();
    }
  int r[3] = {0, 0, 0};
  const bool bias = W->bias != nullptr;
  switch (W->qtype) {
    case MOE_Q_INT4_G128: mfma_residency<MOE_Q_INT4_G128>(bias, gated, block_m, r); break;
    case MOE_Q_NVFP4_G16: mfma_residency<MOE_Q_NVFP4_G16>(bias, gated, block_m, r); break;
    case MOE_Q_INT4ZP_G128: mfma_residency<MOE_Q_INT4ZP_G128>(bias, gated, block_m, r); break;
    case MOE_Q_INT4ZPF_G128: mfma_residency<MOE_Q_INT4ZPF_G128>(bias, gated, block_m, r); break;
    default: mfma_residency<MOE_Q_MXFP4_G32>(bias, gated, block_m, r); break;
  }
  MOE_REQUIRE(r[1] > 0 && r[2] > 0, MOE_EHIP, "moe_gemm_occupancy: the occupancy API gave no answer");
  if (g_res_n < 256) {
    g_res_key[g_res_n] = key;
    for (int j = 0; j < 3; ++j) g_res_val[g_res_n][j] = r[j];
    ++g_res_n;
  }
  for (int j = 0; j < 3; ++j) resident[j] = r[j];
  return ok();
}

extern "C" int moe_w4a16_gemm(const uint16_t* A, int64_t a_rows, int32_t lda, uint16_t* C, int32_t ldc,
                              const moe_weights* W, const int32_t* sorted_token_ids,
                              const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                              int64_t numel, int32_t top_k, int32_t block_m,
                              const moe_gemm_config* cfg, hipStream_t stream) {
  return gemm_impl(kActNone, 0.f, 0.f, A, a_rows, lda, C, ldc, W, sorted_token_ids, expert_ids,
                   num_tokens_post_padded, numel, top_k, block_m, cfg, stream);
}

static int gemm_combine_impl(const uint16_t* A, int64_t a_rows, int32_t lda, uint16_t* y, int32_t ldy,
                             const moe_weights* W, const int32_t* sorted_token_ids, const int32_t* expert_ids,
                             const int32_t* num_tokens_post_padded, int64_t M, int32_t top_k, int32_t block_m,
                             const float* topk_weights, const int32_t* slot_local_ids, float routed_scaling,
                             int32_t* counters, int64_t n_counters, bool noalloc, uint16_t* out, int32_t ldo,
                             const moe_gemm_config* cfg, hipStream_t stream) {
  const char* fn = noalloc ? "moe_w4a16_gemm_combine_noalloc" : "moe_w4a16_gemm_combine";
  MOE_REQUIRE(M >= 0 && M < (1 << 30) && top_k >= 1 && top_k <= 64, MOE_EINVAL,
              "%s: M=%lld top_k=%d", fn, (long long)M, top_k);
  MOE_REQUIRE(W, MOE_EINVAL, "%s: null weights", fn);
  MOE_REQUIRE(!(W->flags & MOE_PREP_GATE_UP), MOE_EINVAL,
              "%s: the weighted sum follows the down projection, not a gate/up pair", fn);
  MOE_REQUIRE(block_m >= 1 && block_m <= 16, MOE_EUNSUPPORTED,
              "%s: block_m=%d outside 1..16 (the streaming decode kernel)", fn, block_m);
  moe_gemm_config c{};
  if (cfg && cfg->kernel != MOE_GEMM_AUTO) {
    c = *cfg;
  } else {
    c = stream_config(W, M * top_k, device_cu_count());  // the fused weighted sum runs in the streaming kernel
  }
  if (noalloc) {
    MOE_REQUIRE(c.ng == 1 || c.ng == 2 || c.ng == 4, MOE_EINVAL, "%s: ng=%d", fn, c.ng);
    const int64_t need = M * ((W->N / kTileN + c.ng - 1) / c.ng);
    MOE_REQUIRE(need <= kNoAllocCounters, MOE_ESIZE,
                "%s: M=%lld tokens x %lld column strips need %lld arrival counters; the library's "
                "scratch holds %lld (use moe_w4a16_gemm_combine with caller counters)",
                fn, (long long)M, (long long)(need / (M > 0 ? M : 1)), (long long)need,
                (long long)kNoAllocCounters);
  }
  if (M == 0) return ok();
  MOE_REQUIRE(topk_weights && slot_local_ids && out && y, MOE_EINVAL, "%s: null pointer", fn);
  MOE_REQUIRE(noalloc || counters, MOE_EINVAL, "%s: null counters", fn);
  MOE_REQUIRE(ldo >= W->N && ((uintptr_t)out & 1) == 0, MOE_EINVAL,
              "%s: ldo=%d below N=%d or misaligned out", fn, ldo, W->N);
  MOE_REQUIRE(((uintptr_t)counters & 3) == 0 && n_counters >= 0, MOE_EINVAL,
              "%s: misaligned counters or negative count", fn);
  if (noalloc) {
    int rc = scratch_counters(&counters);
    if (rc) return rc;
    n_counters = kNoAllocCounters;
  }
  const int64_t numel = M * top_k;
  const CombineSpec cmb{topk_weights, slot_local_ids, out, ldo, counters, n_counters, top_k, M, routed_scaling,
                        noalloc};
  return gemm_impl(kActNone, 0.f, 0.f, A, a_rows, lda, y, ldy, W, sorted_token_ids, expert_ids,
                   num_tokens_post_padded, numel, 1, block_m, &c, stream, nullptr, 0, nullptr, &cmb);
}

extern "C" int moe_w4a16_gemm_combine(const uint16_t* A, int64_t a_rows, int32_t lda, uint16_t* y, int32_t ldy,
                                      const moe_weights* W, const int32_t* sorted_token_ids,
                                      const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                                      int64_t M, int32_t top_k, int32_t block_m, const float* topk_weights,
                                      const int32_t* slot_local_ids, float routed_scaling, int32_t* counters,
                                      int64_t n_counters, uint16_t* out, int32_t ldo,
                                      const moe_gemm_config* cfg, hipStream_t stream) {
  return gemm_combine_impl(A, a_rows, lda, y, ldy, W, sorted_token_ids, expert_ids, num_tokens_post_padded, M,
                           top_k, block_m, topk_weights, slot_local_ids, routed_scaling, counters, n_counters,
                           false, out, ldo, cfg, stream);
}

extern "C" int moe_w4a16_gemm_combine_noalloc(const uint16_t* A, int64_t a_rows, int32_t lda, uint16_t* y,
                                              int32_t ldy, const moe_weights* W, const int32_t* sorted_token_ids,
                                              const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                                              int64_t M, int32_t top_k, int32_t block_m,
                                              const float* topk_weights, const int32_t* slot_local_ids,
                                              float routed_scaling, uint16_t* out, int32_t ldo,
                                              const moe_gemm_config* cfg, hipStream_t stream) {
  return gemm_combine_impl(A, a_rows, lda, y, ldy, W, sorted_token_ids, expert_ids, num_tokens_post_padded, M,
                           top_k, block_m, topk_weights, slot_local_ids, routed_scaling, nullptr, 0, true, out,
                           ldo, cfg, stream);
}

extern "C" int moe_w4a16_gemm_act_routed(moe_act_kind kind, float alpha, float limit, const uint16_t* A,
                                         int64_t a_rows, int32_t lda, uint16_t* out, int32_t ldo,
                                         const moe_weights* W13, const int32_t* topk_ids, int64_t M,
                                         int32_t top_k, int32_t expert_start, int32_t block_m,
                                         int32_t* sorted_token_ids, int32_t* expert_ids,
                                         int32_t* num_tokens_post_padded, int32_t* slot_local_ids,
                                         const moe_gemm_config* cfg, hipStream_t stream) {
  MOE_REQUIRE(kind == MOE_ACT_SILU_MUL || kind == MOE_ACT_SWIGLU_ALPHA || kind == MOE_ACT_RELU2, MOE_EINVAL,
              "moe_w4a16_gemm_act_routed: unknown activation %d", (int)kind);
  MOE_REQUIRE(M >= 0 && top_k >= 1 && top_k <= 64, MOE_EINVAL, "moe_w4a16_gemm_act_routed: M=%lld top_k=%d",
              (long long)M, top_k);
  const int64_t numel = M * top_k;
  MOE_REQUIRE(numel <= kFusedAlignSlots, MOE_EUNSUPPORTED,
              "moe_w4a16_gemm_act_routed: %lld slots; the fused align takes at most %d (use moe_align)",
              (long long)numel, kFusedAlignSlots);
  MOE_REQUIRE(block_m >= 1 && block_m <= 16, MOE_EUNSUPPORTED,
              "moe_w4a16_gemm_act_routed: block_m=%d outside 1..16", block_m);
  MOE_REQUIRE(W13, MOE_EINVAL, "moe_w4a16_gemm_act_routed: null weights");
  MOE_REQUIRE(W13->n_experts >= 1 && W13->n_experts <= 512, MOE_EUNSUPPORTED,
              "moe_w4a16_gemm_act_routed: n_experts=%d outside 1..512", W13->n_experts);
  MOE_REQUIRE(expert_start >= 0, MOE_EINVAL, "moe_w4a16_gemm_act_routed: expert_start=%d", expert_start);
  MOE_REQUIRE(numel == 0 || topk_ids, MOE_EINVAL, "moe_w4a16_gemm_act_routed: null topk_ids");
  int64_t cap = 0, cap_blocks = 0;
  int rc = moe_align_capacity(M, top_k, W13->n_experts, block_m, &cap, &cap_blocks);
  if (rc) return rc;
  // (as moe_align: empty buffers may be NULL)
  MOE_REQUIRE(num_tokens_post_padded && ((sorted_token_ids && expert_ids) || cap == 0) &&
                  (slot_local_ids || numel == 0),
              MOE_EINVAL, "moe_w4a16_gemm_act_routed: null align output");
  if (numel == 0) {  // nothing routed: the align outputs of an empty batch (moe_align writes the same)
    return moe_align(topk_ids, 0, top_k, expert_start, W13->n_experts, block_m, sorted_token_ids, expert_ids,
                     num_tokens_post_padded, slot_local_ids, stream);
  }
  const int act = kind == MOE_ACT_SILU_MUL ? kActSilu : (kind == MOE_ACT_SWIGLU_ALPHA ? kActSwiglu : kActRelu2);
  moe_gemm_config c{};
  if (cfg && cfg->kernel != MOE_GEMM_AUTO) {
    c = *cfg;
  } else {
    c = stream_config(W13, numel, device_cu_count());  // the fused align runs in the streaming kernel
    if (act_paired(act) && c.ng < 2) c.ng = 2;
  }
  return gemm_impl(act, alpha, limit, A, a_rows, lda, out, ldo, W13, sorted_token_ids, expert_ids,
                   num_tokens_post_padded, numel, top_k, block_m, &c, stream, topk_ids, expert_start,
                   slot_local_ids);
}

extern "C" int moe_w4a16_gemm_act(moe_act_kind kind, float alpha, float limit, const uint16_t* A,
                                  int64_t a_rows, int32_t lda, uint16_t* out, int32_t ldo,
                                  const moe_weights* W13, const int32_t* sorted_token_ids,
                                  const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                                  int64_t numel, int32_t top_k, int32_t block_m,
                                  const moe_gemm_config* cfg, hipStream_t stream) {
  MOE_REQUIRE(kind == MOE_ACT_SILU_MUL || kind == MOE_ACT_SWIGLU_ALPHA || kind == MOE_ACT_RELU2, MOE_EINVAL,
              "moe_w4a16_gemm_act: unknown activation %d", (int)kind);
  const int act = kind == MOE_ACT_SILU_MUL ? kActSilu : (kind == MOE_ACT_SWIGLU_ALPHA ? kActSwiglu : kActRelu2);
  return gemm_impl(act, alpha, limit, A, a_rows, lda, out, ldo, W13, sorted_token_ids, expert_ids,
                   num_tokens_post_padded, numel, top_k, block_m, cfg, stream);
}
