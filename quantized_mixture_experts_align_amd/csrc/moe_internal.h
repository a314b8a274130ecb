// Internal helpers shared by the HIP sources of libmoe_w4a16 (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>

#include "moe_w4a16.h"

namespace moe {

// ---------------------------------------------------------------------------- errors
// Sets the thread-local error text and returns `code` (negative moe_status).
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int ok();  // clears the error text, returns MOE_OK
int check_launch(const char* what);  // MOE_EHIP with text if the last launch failed

#define MOE_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) return ::moe::fail(code, __VA_ARGS__); \
  } while (0)

// ---------------------------------------------------------------------------- tiled layout
// A weight tile is 16 output rows x 64 reduction columns of one expert: 512 bytes of codes.
// Lane l (0..63) of a wave owns 8 bytes at offset 8*l: two dwords, dword i holding the eight
// codes of row (l % 16), k = 32*i + 8*(l / 16) + 0..7 (low nibble = even k).  That is exactly
// the A operand of v_mfma_f32_16x16x32_bf16 for k-steps i = 0, 1 (row = output feature), and a
// contiguous 512-byte read for the whole wave.
constexpr int kTileN = 16;
constexpr int kTileK = 64;
constexpr int kTileBytes = kTileN * kTileK / 2;

// the int4 formats: a group of 128 along K spans two 64-column tiles
inline __host__ __device__ bool pair_grouped(int q) {
  return q == MOE_Q_INT4_G128 || q == MOE_Q_INT4ZP_G128 || q == MOE_Q_INT4ZPF_G128;
}
inline __host__ __device__ bool has_zero_points(int q) { return q == MOE_Q_INT4ZP_G128 || q == MOE_Q_INT4ZPF_G128; }
inline __host__ __device__ bool valid_qtype(int q) { return q >= MOE_Q_INT4_G128 && q <= MOE_Q_INT4ZPF_G128; }
inline __host__ __device__ int group_of(int q) { return pair_grouped(q) ? 128 : (q == MOE_Q_NVFP4_G16 ? 16 : 32); }

// Scale bytes per (16-row x 64-column) tile.  NVFP4: 16 rows x 4 e4m3 codes; MXFP4: 16 rows x
// 2 E8M0 codes; int4: the group of 128 spans two tiles, stored per tile pair as 16 bf16;
// asymmetric int4 (both zero-point kinds): per tile pair 16 dwords, each bf16 scale | zero point
// << 16 (the integer 0..15, or the float16 bit pattern).
inline __host__ __device__ int scale_bytes_per_tile(int q) {
  return q == MOE_Q_NVFP4_G16 ? 64 : (q == MOE_Q_MXFP4_G32 ? 32 : (has_zero_points(q) ? 32 : 16));
}
// bytes of scales per scale step of a 16-row tile column: a tile pair (int4 formats) or a tile
inline __host__ __device__ int scale_step_bytes(int q) {
  return pair_grouped(q) ? 2 * scale_bytes_per_tile(q) : scale_bytes_per_tile(q);
}

inline __host__ __device__ size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// moe_w4a16_gemm_combine_noalloc: arrival counters in the library's scratch array per device
constexpr int64_t kNoAllocCounters = MOE_NOALLOC_MAX_COUNTERS;

// act-order (g_idx) weights: most input columns per expert (the grouping is staged in LDS)
constexpr int kMaxActOrderK = 16384;

// MFMA GEMM: align blocks per XCD workgroup group (launch order only, never results).  With a
// short K (<= 1024) a workgroup is brief and an expert's whole weight set fits an XCD's L2, so
// eight consecutive blocks -- mostly one expert's -- share one XCD (measured: int4 layers 5-10%
// faster than with 1).  With a long K the weights stream from HBM: two consecutive 64-slot blocks
// per XCD let a pair share each weight fetch through one L2 (measured: NVFP4 and MXFP4 prefill
// GEMMs 0.5-6% faster than 1, 4 and 8 are slower); 128-slot blocks keep 1.
inline int default_group_m(int K, int block_m) { return K <= 1024 ? 8 : (block_m == 64 ? 2 : 1); }

// Workgroups go to the 8 XCDs round-robin by launch index, and each XCD has its own L2.  The
// MFMA GEMM maps launch index P of a grid of G = nblk * (align blocks) workgroups to a logical
// (align block mb, column block nb) so that workgroups sharing data run on one XCD: a group is
// gm_max consecutive align blocks x all nblk column blocks (column block outer, so the
// workgroups reading the same weight tiles are adjacent; all of them read the group's
// activation rows), and whole groups go round-robin over the XCDs.  The map is a bijection on
// [0, G) (a trailing partial round of groups keeps the identity order; the last group may hold
// fewer than gm_max blocks).
constexpr int kXcds = 8;
__host__ __device__ inline void xcd_grouped_block(int G, int P, int nblk, int gm_max, int& mb, int& nb) {
  const int C = gm_max * nblk;
  const int full = (G / (kXcds * C)) * (kXcds * C);
  int L = P;
  if (P < full) {
    const int x = P % kXcds, j = P / kXcds;
    L = ((j / C) * kXcds + x) * C + j % C;
  }
  const int g = L / C, r = L - g * C;
  const int rest = G / nblk - g * gm_max;
  const int gm = gm_max < rest ? gm_max : rest;
  mb = g * gm_max + r % gm;
  nb = r / gm;
}

// Launch configuration of the streaming decode kernel for about `numel` live slots (the fused
// align and the fused weighted sum run only there).
moe_gemm_config stream_config(const moe_weights* W, int64_t numel, int num_cus);

// ---------------------------------------------------------------------------- device math
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return (uint16_t)(__builtin_bit_cast(uint16_t, (__bf16)f));
}

// ---------------------------------------------------------------------------- activations
// (hardware reciprocal, within 1 ulp: the result is rounded to bf16)
__device__ __forceinline__ float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// silu(gate) * up -- silu_and_mul of the Muse Spark experiment.
struct SiluMul {
  float alpha, limit;
  __device__ __forceinline__ float operator()(float g, float u) const { return g * sigmoid_f(g) * u; }
};
// Non-gated relu(h)^2 (the relu2 activation of the sglang PR 31552 test, is_gated=False).
struct Relu2 {
  float alpha, limit;
  __device__ __forceinline__ float operator()(float h) const {
    const float r = fmaxf(h, 0.0f);
    return r * r;
  }
};
// GPT-OSS: gate clamped from above, up clamped to [-limit, limit], then
// gate * sigmoid(alpha * gate) * (up + 1)  (swiglu_gpt_oss_sigmoid_alpha_contiguous, sglang PR 28231).
struct SwigluAlpha {
  float alpha, limit;
  __device__ __forceinline__ float operator()(float g, float u) const {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
    return g * sigmoid_f(alpha * g) * (u + 1.0f);
  }
};

}  // namespace moe
