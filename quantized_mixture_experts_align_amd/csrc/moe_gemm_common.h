// Shared pieces of the grouped W4A16 GEMM kernels: arguments, group-scale loading and the
// in-register dequantisation of one dword of codes (not part of the ABI).
//
// Weights are in the tiled layout written by moe_w4a16_prepare: 16 rows x 64 columns = 512
// bytes per tile; lane l of a wave reads 8 contiguous bytes, which are the
// v_mfma_f32_16x16x32_bf16 A operand of row l%16 for two k-steps (k = 32 i + 8 (l/16) + 0..7).
#pragma once

#include <algorithm>

#include "moe_internal.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  uint16_t* C;
  int64_t ldc;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gs;
  const uint16_t* bias;
  const int32_t* sorted;
  const int32_t* eids;
  const int32_t* ntpp;
  int32_t numel, top_k, block_m, N, K, E;
  float alpha, limit;  // activation parameters of the fused gate/up epilogue
  int32_t group_m;     // MFMA: align blocks per XCD workgroup group
  // Fused route-and-align (streaming kernel, at most kFusedAlignSlots slots): with topk_ids set,
  // every workgroup computes the align itself instead of reading sorted/eids/ntpp, and
  // workgroup 0 writes the align outputs for the kernels that follow.
  const int32_t* topk_ids;
  int32_t expert_start, cap, cap_blocks;
  int32_t* sorted_out;
  int32_t* eids_out;
  int32_t* ntpp_out;
  int32_t* slot_local_out;
  // Fused top-k weighted sum without norm (streaming kernel, plain projection, top_k = 1 rows):
  // with cmb_out set, the output rows C are still written, and the last item to finish a (token,
  // column strip) sums the token's live rows of that strip into cmb_out.
  const float* cmb_gw;     // [cmb_ntok, cmb_k] top-k weights
  const int32_t* cmb_live; // [cmb_ntok, cmb_k] local expert id of each slot, -1 = dead
  uint16_t* cmb_out;       // [cmb_ntok, cmb_ldo]
  int32_t* cmb_cnt;        // [cmb_ntok, strips] arrival counters: zero on entry, left zero
  int32_t cmb_k, cmb_ntok;
  int64_t cmb_ldo;
  float cmb_rsf;           // routed scaling factor
  // MFMA: block schedule (moe_align_sched), or null for the align order
  const int32_t* border;
};
constexpr int kFusedAlignSlots = 128;  // two 64-slot batches of one wave

// Fused gate/up epilogue: the GEMM's output tiles come in (gate, up) pairs held by the same lane;
// both are rounded to bf16 as the stored GEMM output would be, then the activation is applied
// exactly as moe_act does, so the fused result equals GEMM + moe_act bit for bit.
enum { kActNone = 0, kActSilu = 1, kActSwiglu = 2, kActRelu2 = 3 };
// gated activations pair each gate tile with the up tile I/16 tiles further on
template <int ACT>
constexpr bool act_paired() { return ACT == kActSilu || ACT == kActSwiglu; }
inline bool act_paired(int act) { return act == kActSilu || act == kActSwiglu; }
// the non-gated relu2 epilogue: h rounded to bf16 as the stored GEMM output would be
__device__ __forceinline__ float fused_relu2(float h) { return Relu2{0.f, 0.f}(bf16_to_f32(f32_to_bf16(h))); }
template <int ACT>
__device__ __forceinline__ float fused_act(float gate, float up, const GemmArgs& a) {
  const float g = bf16_to_f32(f32_to_bf16(gate)), u = bf16_to_f32(f32_to_bf16(up));
  if constexpr (ACT == kActSilu) return SiluMul{a.alpha, a.limit}(g, u);
  else return SwigluAlpha{a.alpha, a.limit}(g, u);
}

// ---------------------------------------------------------------------------- dequant
// Group scales of one 64-column tile for this lane, kept as raw bits (they sit in prefetch
// rings) and converted to fp32 at use: s(i, lane) is the scale of k-step i (k = 32 i + 8 (lane/16)
// + 0..7 of the tile); for the int4 formats m(i, lane) is the weight's additive term, -z * s
// (z = 8 for uint4b8), so that a weight is u * s + m.
template <int QT> struct TileScale;

// NVFP4: the row's four e4m3 codes of the tile; k-step i of this lane is group 2 i + lane/32.
template <> struct TileScale<MOE_Q_NVFP4_G16> {
  uint32_t raw;
  static constexpr int kRowBytes = 4;  // scale bytes per row and tile
  __device__ __forceinline__ void load(const uint8_t* tile_scales, int kt, int lane) {
    raw = reinterpret_cast<const uint32_t*>(tile_scales)[(int64_t)kt * 16 + (lane & 15)];
  }
  __device__ __forceinline__ float s(int i, int lane) const {
    return __builtin_amdgcn_cvt_f32_fp8((int)(raw >> (8 * (lane >> 5) + 16 * i)), 0);
  }
  __device__ __forceinline__ float m(int, int) const { return 0.f; }
};
// MXFP4: the row's two E8M0 codes (one per k-step) -> fp32 powers of two (exponent field = code).
template <> struct TileScale<MOE_Q_MXFP4_G32> {
  uint32_t raw;
  static constexpr int kRowBytes = 2;
  __device__ __forceinline__ void load(const uint8_t* tile_scales, int kt, int lane) {
    raw = reinterpret_cast<const uint16_t*>(tile_scales)[(int64_t)kt * 16 + (lane & 15)];
  }
  __device__ __forceinline__ float s(int i, int) const { return __uint_as_float(((raw >> (8 * i)) & 0xFFu) << 23); }
  __device__ __forceinline__ float m(int, int) const { return 0.f; }
};
// int4: one bf16 scale per group of 128 (a tile pair).
template <> struct TileScale<MOE_Q_INT4_G128> {
  uint32_t raw;
  static constexpr int kRowBytes = 2;  // per tile pair
  __device__ __forceinline__ void load(const uint8_t* tile_scales, int kt, int lane) {
    raw = reinterpret_cast<const uint16_t*>(tile_scales)[(int64_t)(kt >> 1) * 16 + (lane & 15)];
  }
  __device__ __forceinline__ float s(int, int) const { return __uint_as_float(raw << 16); }
  __device__ __forceinline__ float m(int i, int lane) const { return -8.0f * s(i, lane); }
};
// asymmetric int4: per row and group of 128 one dword, bf16 scale | zero point << 16.
template <> struct TileScale<MOE_Q_INT4ZP_G128> {
  uint32_t raw;
  static constexpr int kRowBytes = 4;  // per tile pair
  __device__ __forceinline__ void load(const uint8_t* tile_scales, int kt, int lane) {
    raw = reinterpret_cast<const uint32_t*>(tile_scales)[(int64_t)(kt >> 1) * 16 + (lane & 15)];
  }
  __device__ __forceinline__ float s(int, int) const { return __uint_as_float(raw << 16); }
  // -z * s is exact in fp32 (4 x 8 significant bits)
  __device__ __forceinline__ float m(int i, int lane) const { return -(float)((raw >> 16) & 0xFu) * s(i, lane); }
};
// asymmetric int4 with float zero points: per row and group of 128 one dword, bf16 scale |
// float16 zero point << 16.
template <> struct TileScale<MOE_Q_INT4ZPF_G128> {
  uint32_t raw;
  static constexpr int kRowBytes = 4;  // per tile pair
  __device__ __forceinline__ void load(const uint8_t* tile_scales, int kt, int lane) {
    raw = reinterpret_cast<const uint32_t*>(tile_scales)[(int64_t)(kt >> 1) * 16 + (lane & 15)];
  }
  __device__ __forceinline__ float s(int, int) const { return __uint_as_float(raw << 16); }
  // -z * s is exact in fp32 (11 x 8 significant bits)
  __device__ __forceinline__ float m(int i, int lane) const {
    return -(float)__builtin_bit_cast(_Float16, (uint16_t)(raw >> 16)) * s(i, lane);
  }
};

__device__ __forceinline__ uint32_t bits2(bf16x2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Byte B of x as a float (v_cvt_f32_ubyteB).  Written out because the compiler otherwise folds
// the nibble mask into a bit-field extract followed by a byte-0 convert, one instruction more.
template <int B>
__device__ __forceinline__ float ubyte_to_f32(uint32_t x) {
  float r;
  if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
  else if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
  else if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// Eight codes (one dword, k order) -> eight bf16 weights, scale folded in (the MFMA A operand).
// m: the int4 formats' additive term (TileScale::m), unused by the fp4 formats.
template <int QT>
__device__ __forceinline__ u32x4_t dequant8(uint32_t w, float s, float m) {
  u32x4_t o;
  if constexpr (QT == MOE_Q_MXFP4_G32) {
    // the hardware fp4 convert applies a power-of-two scale exactly (its exponent field)
    o[0] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
    o[1] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
    o[2] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
    o[3] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
  } else if constexpr (QT == MOE_Q_NVFP4_G16) {
    // e2m1 * e4m3 has at most 5 significant bits: exact in fp32 and in bf16
    f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    o[0] = pack_bf16x2(p0[0] * s, p0[1] * s);
    o[1] = pack_bf16x2(p1[0] * s, p1[1] * s);
    o[2] = pack_bf16x2(p2[0] * s, p2[1] * s);
    o[3] = pack_bf16x2(p3[0] * s, p3[1] * s);
  } else {
    // int4 formats: u * s + m = (u - z) * s in one fp32 fma (exact for integer zero points: 4 x 8
    // significant bits), rounded to bf16; even-k nibbles are the low nibbles of the four bytes,
    // odd-k the high ones
    static_assert(QT == MOE_Q_INT4_G128 || QT == MOE_Q_INT4ZP_G128 || QT == MOE_Q_INT4ZPF_G128,
                  "unknown weight format");
    const uint32_t t0 = w & 0x0F0F0F0Fu, t1 = (w >> 4) & 0x0F0F0F0Fu;
    const float m8s = m;
    o[0] = pack_bf16x2(fmaf(ubyte_to_f32<0>(t0), s, m8s), fmaf(ubyte_to_f32<0>(t1), s, m8s));
    o[1] = pack_bf16x2(fmaf(ubyte_to_f32<1>(t0), s, m8s), fmaf(ubyte_to_f32<1>(t1), s, m8s));
    o[2] = pack_bf16x2(fmaf(ubyte_to_f32<2>(t0), s, m8s), fmaf(ubyte_to_f32<2>(t1), s, m8s));
    o[3] = pack_bf16x2(fmaf(ubyte_to_f32<3>(t0), s, m8s), fmaf(ubyte_to_f32<3>(t1), s, m8s));
  }
  return o;
}

// Raw codes for the dot-product path: the group scale is applied to the partial sum instead
// (NVFP4), or folded into the exact power-of-two convert (MXFP4), or into the weight (int4).
template <int QT>
__device__ __forceinline__ u32x4_t dequant8_raw(uint32_t w, float s, float m) {
  if constexpr (QT == MOE_Q_NVFP4_G16) {
    u32x4_t o;
    o[0] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    o[1] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    o[2] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    o[3] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
    return o;
  } else {
    return dequant8<QT>(w, s, m);
  }
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         c, false);
}
// (vector elements are copied to scalars first: a bit_cast of a subscripted vector element
// is not an element-wise read)
__device__ __forceinline__ float dot8(u32x4_t a, u32x4_t b, float c) {
  const uint32_t a0 = a.x, a1 = a.y, a2 = a.z, a3 = a.w, b0 = b.x, b1 = b.y, b2 = b.z, b3 = b.w;
  return dot2(a3, b3, dot2(a2, b2, dot2(a1, b1, dot2(a0, b0, c))));
}

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int QT, bool BIAS>
__device__ __forceinline__ float epilogue(float v, const GemmArgs& a, int e, int n) {
  if constexpr (QT == MOE_Q_NVFP4_G16) v *= a.gs[e];
  if constexpr (BIAS) v += bf16_to_f32(a.bias[(int64_t)e * a.N + n]);
  return v;
}

// launchers, one explicit instantiation per weight format (moe_gemm_q*.hip)
template <int QT>
int launch_gemm_decode(bool bias, int act, const GemmArgs& a, const moe_gemm_config& c, int cap_blocks,
                       int num_cus, hipStream_t st);
template <int QT>
int launch_gemm_stream(bool bias, int act, const GemmArgs& a, const moe_gemm_config& c, int cap_blocks,
                       int num_cus, hipStream_t st);
template <int QT>
int launch_gemm_mfma(bool bias, int act, const GemmArgs& a, const moe_gemm_config& c, int cap_blocks,
                     hipStream_t st);
template <int QT>
int mfma_residency(bool bias, bool gated, int block_m, int* resident);
int device_cu_count();

}  // namespace moe
