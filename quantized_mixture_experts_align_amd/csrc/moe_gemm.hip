// Grouped W4A16 GEMM over the align blocks, dequantising 4-bit weights in registers.
//
// The computation is that of moe_wna16_marlin_gemm in the Muse Spark experiment (and the
// Marlin template of the "sglang PR 31552" summary): for each block of sorted slots of one
// expert, C[slot] = dequant(W[e]) . A[slot / top_k] with fp32 accumulation, the per-expert bias
// added at the end (kHasBias there, a template parameter here too) and results in bf16.
//
// Weights use the tiled layout written by moe_w4a16_prepare (16 rows x 64 columns = 512 bytes
// per tile; lane l of a wave reads 8 contiguous bytes = the v_mfma_f32_16x16x32_bf16 A operand
// of row l%16 for two k-steps).  So every weight load is a fully coalesced 512-byte wave read
// straight from HBM into registers, dequantised there, and used as the MFMA A operand (rows =
// output features), with the activations as the B operand (columns = slots).
//
// Two kernels:
//   gemm_decode  block_m <= 16 (decode).  Workgroup = one 16-row weight tile x one align block,
//                its waves splitting K.  Blocks with few live rows use wave dot products
//                (v_dot2_f32_bf16 on raw codes, group scale applied to the partial sum); fuller
//                blocks use one MFMA column of 16 slots.  Partial sums reduced through LDS.
//   gemm_mfma    block_m in {16,32,64,128} (prefill).  Workgroup = 4 waves, each owning NG
//                16-row n-tiles and all 16*MG slots of the block; the activation tile of each
//                64-wide K step is staged in LDS (double buffered) in MFMA B-operand order, so
//                every dequantised weight fragment feeds MG MFMAs.
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
};

// ---------------------------------------------------------------------------- dequant
// Per-lane scale state of one 64-column tile for the two k-steps.
template <int QT> struct TileScale;

// NVFP4: two e4m3 group scales (one per k-step) as fp32.
template <> struct TileScale<MOE_Q_NVFP4_G16> {
  float s[2];
  __device__ __forceinline__ void load(const uint8_t* tile_scales, int kt, int lane) {
    const uint32_t dw = reinterpret_cast<const uint32_t*>(tile_scales)[(int64_t)kt * 16 + (lane & 15)];
    // k-step i covers k = 32 i + 8 (lane/16) + 0..7: group 2 i + (lane / 32) of the tile's four
    const int sh = 8 * (lane >> 5);
    s[0] = __builtin_amdgcn_cvt_f32_fp8((int)(dw >> sh), 0);
    s[1] = __builtin_amdgcn_cvt_f32_fp8((int)(dw >> (sh + 16)), 0);
  }
};
// MXFP4: the E8M0 code of each k-step as an fp32 power of two (exponent field = code).
template <> struct TileScale<MOE_Q_MXFP4_G32> {
  float s[2];
  __device__ __forceinline__ void load(const uint8_t* tile_scales, int kt, int lane) {
    const uint32_t h = reinterpret_cast<const uint16_t*>(tile_scales)[(int64_t)kt * 16 + (lane & 15)];
    s[0] = __uint_as_float((h & 0xFFu) << 23);
    s[1] = __uint_as_float((h >> 8) << 23);
  }
};
// int4: one bf16 scale per group of 128 (a tile pair).
template <> struct TileScale<MOE_Q_INT4_G128> {
  float s[2];
  __device__ __forceinline__ void load(const uint8_t* tile_scales, int kt, int lane) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(tile_scales)[(int64_t)(kt >> 1) * 16 + (lane & 15)];
    s[0] = s[1] = bf16_to_f32(h);
  }
};

__device__ __forceinline__ uint32_t bits2(bf16x2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Eight codes (one dword, k order) -> eight bf16 weights, scale folded in (the MFMA A operand).
template <int QT>
__device__ __forceinline__ u32x4_t dequant8(uint32_t w, float s) {
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
    // uint4b8: (u - 8) * s, exact in fp32 (4 x 8 significant bits), rounded once to bf16
    const uint32_t t0 = w & 0x0F0F0F0Fu, t1 = (w >> 4) & 0x0F0F0F0Fu;
    const float m8s = -8.0f * s;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = pack_bf16x2(fmaf((float)((t0 >> (8 * j)) & 0xFFu), s, m8s),
                         fmaf((float)((t1 >> (8 * j)) & 0xFFu), s, m8s));
  }
  return o;
}

// Raw codes for the dot-product path: the group scale is applied to the partial sum instead
// (NVFP4), or folded into the exact power-of-two convert (MXFP4), or into the weight (int4).
template <int QT>
__device__ __forceinline__ u32x4_t dequant8_raw(uint32_t w, float s) {
  if constexpr (QT == MOE_Q_NVFP4_G16) {
    u32x4_t o;
    o[0] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    o[1] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    o[2] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    o[3] = bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
    return o;
  } else {
    return dequant8<QT>(w, s);
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

// ---------------------------------------------------------------------------- decode kernel
constexpr int kGemvMax = 4;

template <int QT, bool BIAS, int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void gemm_decode_kernel(GemmArgs a, int gemv_rows) {
  extern __shared__ u32x4_t x_lds[];  // [gemv_rows][K / 8] activations of the dot-product path
  __shared__ int s_rows[16];
  __shared__ int s_cnt;
  __shared__ f32x4_t red[KSPLIT > 1 ? KSPLIT - 1 : 1][64];

  const int nt = blockIdx.x, b = blockIdx.y, B = a.block_m;
  if (b * B >= *a.ntpp) return;
  const int e = a.eids[b];
  if (e < 0 || e >= a.E) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  if (w == 0) {
    const int s = lane < B ? a.sorted[(int64_t)b * B + lane] : a.numel;
    const bool live = s >= 0 && s < a.numel;
    const uint64_t m = __ballot(live);
    if (live) s_rows[__popcll(m & ((1ull << lane) - 1))] = s;
    if (lane == 0) s_cnt = __popcll(m);
  }
  __syncthreads();
  const int cnt = s_cnt;
  if (cnt == 0) return;

  const int NT = a.N / kTileN, KT = a.K / kTileK;
  const int64_t tile0 = ((int64_t)e * NT + nt) * KT;
  const u32x2_t* wp = reinterpret_cast<const u32x2_t*>(a.codes + tile0 * kTileBytes) + lane;
  const uint8_t* sp = a.scales + (QT == MOE_Q_INT4_G128 ? ((int64_t)e * NT + nt) * (KT / 2) * 32
                                                        : tile0 * scale_bytes_per_tile(QT));
  const int kt0 = KT * w / KSPLIT, kt1 = KT * (w + 1) / KSPLIT;
  const int j8 = 8 * (lane >> 4);  // this lane's column offset inside a 32-wide k-step
  constexpr int U = 4;

  if (cnt <= gemv_rows) {
    // ---- dot-product path: activations of the live rows staged in LDS
    const int kc = a.K / 8;
    for (int i = tid; i < cnt * kc; i += 64 * KSPLIT) {
      const int r = i / kc, c = i - r * kc;
      x_lds[i] = *reinterpret_cast<const u32x4_t*>(a.A + (int64_t)(s_rows[r] / a.top_k) * a.lda + c * 8);
    }
    __syncthreads();
    float acc[kGemvMax] = {0.f, 0.f, 0.f, 0.f};
    for (int kt = kt0; kt < kt1; kt += U) {
      u32x2_t q[U];
      TileScale<QT> sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (kt + u < kt1) {
          q[u] = wp[(int64_t)(kt + u) * 64];
          sc[u].load(sp, kt + u, lane);
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (kt + u >= kt1) break;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const u32x4_t wv = dequant8_raw<QT>(q[u][i], sc[u].s[i]);
          const int col = ((kt + u) * kTileK + 32 * i + j8) >> 3;
#pragma unroll
          for (int r = 0; r < kGemvMax; ++r) {
            if (r >= cnt) break;
            const u32x4_t xv = x_lds[r * kc + col];
            if constexpr (QT == MOE_Q_NVFP4_G16)
              acc[r] = fmaf(sc[u].s[i], dot8(wv, xv, 0.f), acc[r]);
            else
              acc[r] = dot8(wv, xv, acc[r]);
          }
        }
      }
    }
    // lanes l, l+16, l+32, l+48 hold the same output row
#pragma unroll
    for (int r = 0; r < kGemvMax; ++r) {
      acc[r] += __shfl_xor(acc[r], 16);
      acc[r] += __shfl_xor(acc[r], 32);
    }
    if constexpr (KSPLIT > 1) {
      if (w > 0 && lane < 16) red[w - 1][lane] = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
      __syncthreads();
      if (w == 0 && lane < 16)
        for (int v = 0; v < KSPLIT - 1; ++v) {
          const f32x4_t o = red[v][lane];
          acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
        }
    }
    if (w == 0 && lane < 16) {
      const int n = nt * kTileN + lane;
#pragma unroll
      for (int r = 0; r < kGemvMax; ++r) {
        if (r >= cnt) break;
        a.C[(int64_t)s_rows[r] * a.ldc + n] = f32_to_bf16(epilogue<QT, BIAS>(acc[r], a, e, n));
      }
    }
    return;
  }

  // ---- MFMA path: one 16-slot column, activations read from global (L2) per k-step
  const int m = lane & 15;
  const bool mrow = m < cnt;
  const uint16_t* xrow = a.A + (int64_t)(mrow ? s_rows[m] / a.top_k : 0) * a.lda + j8;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int kt = kt0; kt < kt1; kt += U) {
    u32x2_t q[U];
    TileScale<QT> sc[U];
    u32x4_t xv[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (kt + u < kt1) {
        q[u] = wp[(int64_t)(kt + u) * 64];
        sc[u].load(sp, kt + u, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          xv[u][i] = mrow ? *reinterpret_cast<const u32x4_t*>(xrow + (kt + u) * kTileK + 32 * i)
                          : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kt + u >= kt1) break;
#pragma unroll
      for (int i = 0; i < 2; ++i) acc = mfma(dequant8<QT>(q[u][i], sc[u].s[i]), xv[u][i], acc);
    }
  }
  if constexpr (KSPLIT > 1) {
    if (w > 0) red[w - 1][lane] = acc;
    __syncthreads();
    if (w == 0)
      for (int v = 0; v < KSPLIT - 1; ++v) acc += red[v][lane];
  }
  if (w == 0 && mrow) {
    // D[n][m]: this lane holds rows n = 4 (lane/16) + 0..3 of column m
    const int n0 = nt * kTileN + 4 * (lane >> 4);
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = epilogue<QT, BIAS>(acc[q], a, e, n0 + q);
    *reinterpret_cast<u32x2_t*>(a.C + (int64_t)s_rows[m] * a.ldc + n0) =
        u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

// ---------------------------------------------------------------------------- MFMA kernel
template <int QT, bool BIAS, int MG, int NG>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmArgs a) {
  constexpr int BM = 16 * MG;
  constexpr int FRAGS = 2 * MG * 64;                 // 16-byte activation fragments per K step
  constexpr int LOADS = FRAGS >= 256 ? FRAGS / 256 : 1;
  __shared__ u32x4_t xs[2][FRAGS];
  __shared__ int s_crow[BM];

  const int NT = a.N / kTileN, KT = a.K / kTileK;
  const int nblk = (NT + 4 * NG - 1) / (4 * NG);
  const int mb = blockIdx.x / nblk, nb = blockIdx.x - mb * nblk;
  if (mb * BM >= *a.ntpp) return;
  const int e = a.eids[mb];
  if (e < 0 || e >= a.E) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;

  if (tid < BM) {
    const int s = a.sorted[(int64_t)mb * BM + tid];
    s_crow[tid] = (s >= 0 && s < a.numel) ? s : -1;
  }
  __syncthreads();

  // activation loader: fragment f -> k-step i, m-group g, MFMA lane fl (row g*16 + fl%16,
  // columns 32 i + 8 (fl / 16) + 0..7 of the K step); LDS slot f, i.e. B-operand order
  const uint16_t* xsrc[LOADS];
  bool xok[LOADS];
#pragma unroll
  for (int l = 0; l < LOADS; ++l) {
    const int f = l * 256 + tid;
    const int fl = f & 63, g = (f >> 6) % MG, i = (f >> 6) / MG;
    const int row = s_crow[g * 16 + (fl & 15)];
    xok[l] = f < FRAGS && row >= 0;
    xsrc[l] = a.A + (int64_t)(row >= 0 ? row / a.top_k : 0) * a.lda + 32 * i + 8 * (fl >> 4);
  }
  u32x4_t xr[LOADS];
  auto load_x = [&](int kt) {
#pragma unroll
    for (int l = 0; l < LOADS; ++l)
      xr[l] = xok[l] ? *reinterpret_cast<const u32x4_t*>(xsrc[l] + kt * kTileK) : u32x4_t{0u, 0u, 0u, 0u};
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int l = 0; l < LOADS; ++l)
      if (l * 256 + tid < FRAGS) xs[buf][l * 256 + tid] = xr[l];
  };

  // weights of this wave: NG consecutive 16-row tiles (clamped for loads at the N edge)
  int ntile[NG];
  bool nok[NG];
  const u32x2_t* wp[NG];
  const uint8_t* sp[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int t = nb * 4 * NG + w * NG + g;
    nok[g] = t < NT;
    ntile[g] = nok[g] ? t : NT - 1;
    const int64_t tile0 = ((int64_t)e * NT + ntile[g]) * KT;
    wp[g] = reinterpret_cast<const u32x2_t*>(a.codes + tile0 * kTileBytes) + lane;
    sp[g] = a.scales + (QT == MOE_Q_INT4_G128 ? ((int64_t)e * NT + ntile[g]) * (KT / 2) * 32
                                              : tile0 * scale_bytes_per_tile(QT));
  }
  u32x2_t wq[NG];
  TileScale<QT> wsc[NG];
  auto load_w = [&](int kt) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      wq[g] = wp[g][(int64_t)kt * 64];
      wsc[g].load(sp[g], kt, lane);
    }
  };

  f32x4_t acc[NG][MG];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int h = 0; h < MG; ++h) acc[g][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_x(0);
  store_x(0);
  load_w(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    u32x2_t cq[NG];
    TileScale<QT> csc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      cq[g] = wq[g];
      csc[g] = wsc[g];
    }
    if (kt + 1 < KT) {
      load_x(kt + 1);
      load_w(kt + 1);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4_t af[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) af[g] = dequant8<QT>(cq[g][i], csc[g].s[i]);
#pragma unroll
      for (int h = 0; h < MG; ++h) {
        const u32x4_t bf = xs[buf][(i * MG + h) * 64 + lane];
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g][h] = mfma(af[g], bf, acc[g][h]);
      }
    }
    if (kt + 1 < KT) store_x(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds D[n = 4 (lane/16) + q][m = lane % 16] of each (n-tile, m-group)
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (!nok[g]) continue;
    const int n0 = ntile[g] * kTileN + 4 * (lane >> 4);
    float gsv = 1.f;
    if constexpr (QT == MOE_Q_NVFP4_G16) gsv = a.gs[e];
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BIAS) {
      const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(a.bias + (int64_t)e * a.N + n0);
      bv[0] = bf16_lo(bb[0]); bv[1] = bf16_hi(bb[0]); bv[2] = bf16_lo(bb[1]); bv[3] = bf16_hi(bb[1]);
    }
#pragma unroll
    for (int h = 0; h < MG; ++h) {
      const int row = s_crow[h * 16 + (lane & 15)];
      if (row < 0) continue;
      const f32x4_t v = acc[g][h];
      float o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = v[q] * gsv + bv[q];
      *reinterpret_cast<u32x2_t*>(a.C + (int64_t)row * a.ldc + n0) =
          u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
  }
}

// ---------------------------------------------------------------------------- dispatch
template <int QT, bool BIAS>
static int launch_decode(const GemmArgs& a, const moe_gemm_config& c, int blocks, hipStream_t st) {
  const dim3 grid(a.N / kTileN, blocks);
  const size_t lds = (size_t)c.gemv_rows * a.K * 2;
  switch (c.ksplit) {
    case 1: hipLaunchKernelGGL((gemm_decode_kernel<QT, BIAS, 1>), grid, dim3(64), lds, st, a, c.gemv_rows); break;
    case 2: hipLaunchKernelGGL((gemm_decode_kernel<QT, BIAS, 2>), grid, dim3(128), lds, st, a, c.gemv_rows); break;
    case 4: hipLaunchKernelGGL((gemm_decode_kernel<QT, BIAS, 4>), grid, dim3(256), lds, st, a, c.gemv_rows); break;
    default: return fail(MOE_EINVAL, "moe_w4a16_gemm: ksplit=%d (1, 2 or 4)", c.ksplit);
  }
  return check_launch("moe_w4a16_gemm (decode)");
}

template <int QT, bool BIAS, int MG>
static int launch_mfma_mg(const GemmArgs& a, int ng, int blocks, hipStream_t st) {
  const int NT = a.N / kTileN;
  const int nblk = (NT + 4 * ng - 1) / (4 * ng);
  const dim3 grid((unsigned)((int64_t)nblk * blocks));
  switch (ng) {
    case 1: hipLaunchKernelGGL((gemm_mfma_kernel<QT, BIAS, MG, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((gemm_mfma_kernel<QT, BIAS, MG, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((gemm_mfma_kernel<QT, BIAS, MG, 4>), grid, dim3(256), 0, st, a); break;
    default: return fail(MOE_EINVAL, "moe_w4a16_gemm: ng=%d (1, 2 or 4)", ng);
  }
  return check_launch("moe_w4a16_gemm (mfma)");
}

template <int QT, bool BIAS>
static int launch_mfma(const GemmArgs& a, const moe_gemm_config& c, int blocks, hipStream_t st) {
  switch (a.block_m) {
    case 16: return launch_mfma_mg<QT, BIAS, 1>(a, c.ng, blocks, st);
    case 32: return launch_mfma_mg<QT, BIAS, 2>(a, c.ng, blocks, st);
    case 64: return launch_mfma_mg<QT, BIAS, 4>(a, c.ng, blocks, st);
    case 128: return launch_mfma_mg<QT, BIAS, 8>(a, c.ng, blocks, st);
    default: return fail(MOE_EUNSUPPORTED, "moe_w4a16_gemm: MFMA kernel needs block_m 16/32/64/128, got %d", a.block_m);
  }
}

template <int QT, bool BIAS>
static int launch(const GemmArgs& a, const moe_gemm_config& c, int blocks, hipStream_t st) {
  if (c.kernel == MOE_GEMM_DECODE) return launch_decode<QT, BIAS>(a, c, blocks, st);
  return launch_mfma<QT, BIAS>(a, c, blocks, st);
}

template <int QT>
static int launch_q(const GemmArgs& a, const moe_gemm_config& c, int blocks, hipStream_t st) {
  return a.bias ? launch<QT, true>(a, c, blocks, st) : launch<QT, false>(a, c, blocks, st);
}

static bool al(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

}  // namespace moe

using namespace moe;

extern "C" int moe_w4a16_gemm(const uint16_t* A, int64_t a_rows, int32_t lda, uint16_t* C, int32_t ldc,
                              const moe_weights* W, const int32_t* sorted_token_ids,
                              const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                              int64_t numel, int32_t top_k, int32_t block_m,
                              const moe_gemm_config* cfg, hipStream_t stream) {
  MOE_REQUIRE(W, MOE_EINVAL, "moe_w4a16_gemm: null weights");
  MOE_REQUIRE(W->qtype >= 0 && W->qtype <= 2, MOE_EINVAL, "moe_w4a16_gemm: bad qtype %d", W->qtype);
  MOE_REQUIRE(W->n_experts >= 1 && W->N >= kTileN && W->N % kTileN == 0 && W->K >= kTileK &&
                  W->K % kTileK == 0,
              MOE_EINVAL, "moe_w4a16_gemm: weights E=%d N=%d K=%d not in the prepared layout",
              W->n_experts, W->N, W->K);
  MOE_REQUIRE(W->codes && W->scales, MOE_EINVAL, "moe_w4a16_gemm: weights without codes/scales");
  MOE_REQUIRE(W->qtype != MOE_Q_NVFP4_G16 || W->global_scale, MOE_EINVAL,
              "moe_w4a16_gemm: NVFP4 weights without global scales");
  MOE_REQUIRE(numel >= 0 && numel < (1 << 30), MOE_EUNSUPPORTED, "moe_w4a16_gemm: numel=%lld", (long long)numel);
  MOE_REQUIRE(top_k >= 1 && block_m >= 1, MOE_EINVAL, "moe_w4a16_gemm: top_k=%d block_m=%d", top_k, block_m);
  MOE_REQUIRE(a_rows >= (numel + top_k - 1) / top_k, MOE_EINVAL,
              "moe_w4a16_gemm: A has %lld rows, slots need %lld", (long long)a_rows,
              (long long)((numel + top_k - 1) / top_k));
  MOE_REQUIRE(lda >= W->K && lda % 8 == 0 && ldc >= W->N && ldc % 4 == 0, MOE_EINVAL,
              "moe_w4a16_gemm: lda=%d (>= K=%d, multiple of 8) ldc=%d (>= N=%d, multiple of 4)", lda,
              W->K, ldc, W->N);
  if (numel == 0) return ok();
  MOE_REQUIRE(A && C && sorted_token_ids && expert_ids && num_tokens_post_padded, MOE_EINVAL,
              "moe_w4a16_gemm: null pointer");
  MOE_REQUIRE(al(A, 16) && al(C, 8) && al(W->codes, 16) && al(W->scales, 4) && (!W->bias || al(W->bias, 8)),
              MOE_EUNSUPPORTED, "moe_w4a16_gemm: misaligned pointer (A 16 B, C 8 B, bias 8 B)");
  moe_gemm_config c{};
  if (cfg && cfg->kernel != MOE_GEMM_AUTO) {
    c = *cfg;
  } else {
    int rc = moe_gemm_choose(W, numel, block_m, 0, &c);
    if (rc) return rc;
    if (cfg) {  // AUTO with explicit knobs: keep the caller's non-zero ones
      if (cfg->ng) c.ng = cfg->ng;
      if (cfg->ksplit) c.ksplit = cfg->ksplit;
    }
  }
  int64_t cap = 0, cap_blocks = 0;
  int rc = moe_align_capacity(numel, 1, W->n_experts, block_m, &cap, &cap_blocks);
  if (rc) return rc;
  MOE_REQUIRE(cap_blocks <= 65535 || c.kernel == MOE_GEMM_MFMA, MOE_EUNSUPPORTED,
              "moe_w4a16_gemm: too many blocks for the decode grid");
  if (c.kernel == MOE_GEMM_DECODE) {
    MOE_REQUIRE(block_m <= 16, MOE_EUNSUPPORTED, "moe_w4a16_gemm: decode kernel needs block_m <= 16");
    MOE_REQUIRE(c.gemv_rows >= 0 && c.gemv_rows <= kGemvMax, MOE_EINVAL, "moe_w4a16_gemm: gemv_rows=%d",
                c.gemv_rows);
    MOE_REQUIRE((int64_t)c.gemv_rows * W->K * 2 <= 65536, MOE_EUNSUPPORTED,
                "moe_w4a16_gemm: gemv_rows=%d x K=%d does not fit the LDS budget", c.gemv_rows, W->K);
  } else {
    MOE_REQUIRE(c.kernel == MOE_GEMM_MFMA, MOE_EINVAL, "moe_w4a16_gemm: unknown kernel %d", c.kernel);
    MOE_REQUIRE((int64_t)((W->N / kTileN + 4 * c.ng - 1) / (4 * std::max(c.ng, 1))) * cap_blocks < (1ll << 31),
                MOE_EUNSUPPORTED, "moe_w4a16_gemm: grid too large");
  }
  GemmArgs a{A, lda, C, ldc,
             static_cast<const uint8_t*>(W->codes), static_cast<const uint8_t*>(W->scales),
             W->global_scale, W->bias, sorted_token_ids, expert_ids, num_tokens_post_padded,
             (int32_t)numel, top_k, block_m, W->N, W->K, W->n_experts};
  switch (W->qtype) {
    case MOE_Q_INT4_G128: return launch_q<MOE_Q_INT4_G128>(a, c, (int)cap_blocks, stream);
    case MOE_Q_NVFP4_G16: return launch_q<MOE_Q_NVFP4_G16>(a, c, (int)cap_blocks, stream);
    default: return launch_q<MOE_Q_MXFP4_G32>(a, c, (int)cap_blocks, stream);
  }
}
