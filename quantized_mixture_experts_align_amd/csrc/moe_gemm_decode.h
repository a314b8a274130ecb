// gemm_decode: grouped W4A16 GEMM for align blocks of at most 16 slots (decode batches),
// where the cost is streaming the touched experts' weights from HBM.
//
// Work item = (live align block, strip of NG 16-row weight tiles).  The grid is persistent: each
// workgroup reads num_tokens_post_padded and walks a contiguous range of the live items, so no
// workgroup is launched for padding capacity.  The KS waves of a workgroup split K; each wave
// streams its NG tiles (512-B coalesced wave loads, two batches of P steps in flight) and:
//   * if the block has at most gemv_rows live slots: dot products (v_dot2_f32_bf16) of the
//     converted codes with the slots' activations, staged once per block in LDS and reused by
//     all NG tiles; the NVFP4 group scale multiplies the 8-element partial sum, the MXFP4
//     power-of-two scale is folded into the fp4 convert, int4 uses (u - 8) * s;
//   * otherwise one MFMA column of 16 slots per tile (activations read from L2 per step).
// Partial sums of the waves are added through LDS in a fixed order (reproducible results).
// With ACT (fused gate/up epilogue) a strip is NG/2 gate tiles plus the matching up tiles.
#pragma once

#include "moe_gemm_common.h"

namespace moe {

constexpr int kGemvMax = 4;
constexpr int kP = 2;  // K steps per prefetch batch

template <int QT, bool BIAS, int NG, int KS, int ACT>
__global__ __launch_bounds__(64 * KS) void gemm_decode_kernel(GemmArgs a, int gemv_rows) {
  static_assert(!act_paired<ACT>() || NG % 2 == 0, "the fused gated epilogue pairs gate and up tiles");
  constexpr int NGA = act_paired<ACT>() ? NG / 2 : NG;
  extern __shared__ u32x4_t x_lds[];  // [gemv_rows][K / 8] activations of the dot-product path
  __shared__ int s_rows[16];
  __shared__ int s_cnt, s_e;
  __shared__ f32x4_t red[KS > 1 ? KS - 1 : 1][NG][64];

  // the wave index is uniform: keep it (and every LDS address derived from it) in scalar registers
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int NT = a.N / kTileN, KT = a.K / kTileK, kc = a.K / 8;
  const int NTA = act_paired<ACT>() ? NT / 2 : NT;  // tiles to assign (gate tiles if fused)
  const int NS = (NTA + NGA - 1) / NGA;
  const int B = a.block_m;
  const int items = (*a.ntpp / B) * NS;
  const int per = (items + (int)gridDim.x - 1) / (int)gridDim.x;
  const int i0 = (int)blockIdx.x * per, i1 = min(items, i0 + per);
  const int kt0 = KT * w / KS, kt1 = KT * (w + 1) / KS;
  const int j8 = 8 * (lane >> 4);
  int cur_b = -1, cnt = 0, e = -1;

  for (int it = i0; it < i1; ++it) {
    const int b = it / NS, strip = it - b * NS;
    if (b != cur_b) {  // new align block: its live slots, expert and (dot path) activations
      __syncthreads();
      if (w == 0) {
        const int s = lane < B ? a.sorted[(int64_t)b * B + lane] : a.numel;
        const bool live = s >= 0 && s < a.numel;
        const uint64_t m = __ballot(live);
        if (live) s_rows[__popcll(m & ((1ull << lane) - 1))] = s;
        if (lane == 0) {
          s_cnt = __popcll(m);
          s_e = a.eids[b];
        }
      }
      __syncthreads();
      cnt = s_cnt;
      e = s_e;
      cur_b = b;
      if (cnt > 0 && cnt <= gemv_rows) {
        for (int i = tid; i < cnt * kc; i += 64 * KS) {
          const int r = i / kc, c = i - r * kc;
          x_lds[i] = *reinterpret_cast<const u32x4_t*>(a.A + (int64_t)(s_rows[r] / a.top_k) * a.lda + c * 8);
        }
        __syncthreads();
      }
    }
    if (cnt == 0 || e < 0 || e >= a.E) continue;

    int tile[NG];
    const u32x2_t* wp[NG];
    const uint8_t* sp[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      tile[g] = g < NGA ? min(strip * NGA + g, NTA - 1) : tile[g - NGA] + NTA;
      const int64_t tile0 = ((int64_t)e * NT + tile[g]) * KT;
      wp[g] = reinterpret_cast<const u32x2_t*>(a.codes + tile0 * kTileBytes) + lane;
      sp[g] = a.scales + ((int64_t)e * NT + tile[g]) * (pair_grouped(QT) ? KT / 2 : KT) * scale_step_bytes(QT);
    }
    const bool gemv = cnt <= gemv_rows;
    const int m = lane & 15;
    const uint16_t* xrow = a.A + (int64_t)(s_rows[m < cnt ? m : 0] / a.top_k) * a.lda + j8;

    u32x2_t q[2][kP][NG];
    TileScale<QT> sc[2][kP][NG];
    u32x4_t xv[2][kP][2];
    auto issue = [&](int slot, int k0) {
#pragma unroll
      for (int u = 0; u < kP; ++u)
        if (k0 + u < kt1) {
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            q[slot][u][g] = wp[g][(int64_t)(k0 + u) * 64];
            sc[slot][u][g].load(sp[g], k0 + u, lane);
          }
          if (!gemv) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
              xv[slot][u][i] = *reinterpret_cast<const u32x4_t*>(xrow + (k0 + u) * kTileK + 32 * i);
          }
        }
    };

    float dacc[NG][kGemvMax];
    f32x4_t macc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      macc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < kGemvMax; ++r) dacc[g][r] = 0.f;
    }
    auto compute = [&](int slot, int k0) {
#pragma unroll
      for (int u = 0; u < kP; ++u) {
        if (k0 + u >= kt1) break;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (gemv) {
            const int col = ((k0 + u) * kTileK + 32 * i + j8) >> 3;
            u32x4_t xr[kGemvMax];
#pragma unroll
            for (int r = 0; r < kGemvMax; ++r)
              if (r < cnt) xr[r] = x_lds[r * kc + col];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
              const float s = sc[slot][u][g].s(i, lane);
              const u32x4_t wv = dequant8_raw<QT>(q[slot][u][g][i], s, sc[slot][u][g].m(i, lane));
#pragma unroll
              for (int r = 0; r < kGemvMax; ++r) {
                if (r >= cnt) break;
                if constexpr (QT == MOE_Q_NVFP4_G16)
                  dacc[g][r] = fmaf(s, dot8(wv, xr[r], 0.f), dacc[g][r]);
                else
                  dacc[g][r] = dot8(wv, xr[r], dacc[g][r]);
              }
            }
          } else {
#pragma unroll
            for (int g = 0; g < NG; ++g)
              macc[g] = mfma(dequant8<QT>(q[slot][u][g][i], sc[slot][u][g].s(i, lane), sc[slot][u][g].m(i, lane)),
                             xv[slot][u][i], macc[g]);
          }
        }
      }
    };

    // two batches in flight: issue batch n+1, then compute batch n
    issue(0, kt0);
    for (int k0 = kt0; k0 < kt1; k0 += 2 * kP) {
      if (k0 + kP < kt1) issue(1, k0 + kP);
      compute(0, k0);
      if (k0 + kP >= kt1) break;
      if (k0 + 2 * kP < kt1) issue(0, k0 + 2 * kP);
      compute(1, k0 + kP);
    }

    // reduce over the waves (fixed order), wave 0 writes
    if (gemv) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int r = 0; r < kGemvMax; ++r) {  // lanes l, l+16, l+32, l+48 hold the same output row
          dacc[g][r] += __shfl_xor(dacc[g][r], 16);
          dacc[g][r] += __shfl_xor(dacc[g][r], 32);
        }
      if constexpr (KS > 1) {
        if (w > 0 && lane < 16)
#pragma unroll
          for (int g = 0; g < NG; ++g) red[w - 1][g][lane] = f32x4_t{dacc[g][0], dacc[g][1], dacc[g][2], dacc[g][3]};
        __syncthreads();
        if (w == 0 && lane < 16)
          for (int v = 0; v < KS - 1; ++v)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
              const f32x4_t o = red[v][g][lane];
              dacc[g][0] += o[0]; dacc[g][1] += o[1]; dacc[g][2] += o[2]; dacc[g][3] += o[3];
            }
      }
      if (w == 0 && lane < 16) {
#pragma unroll
        for (int g = 0; g < NGA; ++g) {
          if (strip * NGA + g >= NTA) break;
          const int n = tile[g] * kTileN + lane;
#pragma unroll
          for (int r = 0; r < kGemvMax; ++r) {
            if (r >= cnt) break;
            float v = epilogue<QT, BIAS>(dacc[g][r], a, e, n);
            if constexpr (act_paired<ACT>())
              v = fused_act<ACT>(v, epilogue<QT, BIAS>(dacc[g + NGA][r], a, e, tile[g + NGA] * kTileN + lane), a);
            else if constexpr (ACT == kActRelu2)
              v = fused_relu2(v);
            a.C[(int64_t)s_rows[r] * a.ldc + n] = f32_to_bf16(v);
          }
        }
      }
    } else {
      if constexpr (KS > 1) {
        if (w > 0)
#pragma unroll
          for (int g = 0; g < NG; ++g) red[w - 1][g][lane] = macc[g];
        __syncthreads();
        if (w == 0)
          for (int v = 0; v < KS - 1; ++v)
#pragma unroll
            for (int g = 0; g < NG; ++g) macc[g] += red[v][g][lane];
      }
      if (w == 0 && m < cnt) {
        // D[n][m]: this lane holds rows n = 4 (lane/16) + 0..3 of column m
#pragma unroll
        for (int g = 0; g < NGA; ++g) {
          if (strip * NGA + g >= NTA) break;
          const int n0 = tile[g] * kTileN + 4 * (lane >> 4);
          float v[4];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            v[qq] = epilogue<QT, BIAS>(macc[g][qq], a, e, n0 + qq);
            if constexpr (act_paired<ACT>())
              v[qq] = fused_act<ACT>(v[qq], epilogue<QT, BIAS>(macc[g + NGA][qq], a, e, tile[g + NGA] * kTileN + 4 * (lane >> 4) + qq), a);
            else if constexpr (ACT == kActRelu2)
              v[qq] = fused_relu2(v[qq]);
          }
          *reinterpret_cast<u32x2_t*>(a.C + (int64_t)s_rows[m] * a.ldc + n0) =
              u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    }
    if constexpr (KS > 1) __syncthreads();  // red[] is reused by the next item
  }
}

template <int QT, bool BIAS, int NG, int ACT>
static int launch_ng(const GemmArgs& a, const moe_gemm_config& c, int grid, hipStream_t st) {
  const size_t lds = (size_t)c.gemv_rows * a.K * 2;
  switch (c.ksplit) {
    case 1: hipLaunchKernelGGL((gemm_decode_kernel<QT, BIAS, NG, 1, ACT>), dim3(grid), dim3(64), lds, st, a, c.gemv_rows); break;
    case 2: hipLaunchKernelGGL((gemm_decode_kernel<QT, BIAS, NG, 2, ACT>), dim3(grid), dim3(128), lds, st, a, c.gemv_rows); break;
    case 4: hipLaunchKernelGGL((gemm_decode_kernel<QT, BIAS, NG, 4, ACT>), dim3(grid), dim3(256), lds, st, a, c.gemv_rows); break;
    default: return fail(MOE_EINVAL, "moe_w4a16_gemm: ksplit=%d (1, 2 or 4)", c.ksplit);
  }
  return check_launch("moe_w4a16_gemm (decode)");
}

template <int QT, bool BIAS, int ACT>
static int launch_decode_b(const GemmArgs& a, const moe_gemm_config& c, int grid, hipStream_t st) {
  if constexpr (!act_paired<ACT>()) {
    if (c.ng == 1) return launch_ng<QT, BIAS, 1, ACT>(a, c, grid, st);
  }
  switch (c.ng) {
    case 2: return launch_ng<QT, BIAS, 2, ACT>(a, c, grid, st);
    case 4: return launch_ng<QT, BIAS, 4, ACT>(a, c, grid, st);
    default: return fail(MOE_EINVAL, "moe_w4a16_gemm: decode ng=%d (1, 2 or 4; 2 or 4 with a fused gated activation)", c.ng);
  }
}

template <int QT>
int launch_gemm_decode(bool bias, int act, const GemmArgs& a, const moe_gemm_config& c, int cap_blocks,
                       int num_cus, hipStream_t st) {
  const int NT = a.N / kTileN;
  const int nta = act_paired(act) ? NT / 2 : NT, nga = act_paired(act) ? c.ng / 2 : c.ng;
  const int ns = (nta + nga - 1) / std::max(nga, 1);
  // persistent grid: enough workgroups to keep every CU streaming, never more than the items
  const int64_t max_items = (int64_t)cap_blocks * ns;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(max_items, (int64_t)num_cus * (16 / c.ksplit)));
  switch (act) {
    case kActNone:
      return bias ? launch_decode_b<QT, true, kActNone>(a, c, grid, st) : launch_decode_b<QT, false, kActNone>(a, c, grid, st);
    case kActSilu:
      return bias ? launch_decode_b<QT, true, kActSilu>(a, c, grid, st) : launch_decode_b<QT, false, kActSilu>(a, c, grid, st);
    case kActRelu2:
      return bias ? launch_decode_b<QT, true, kActRelu2>(a, c, grid, st) : launch_decode_b<QT, false, kActRelu2>(a, c, grid, st);
    default:
      return bias ? launch_decode_b<QT, true, kActSwiglu>(a, c, grid, st) : launch_decode_b<QT, false, kActSwiglu>(a, c, grid, st);
  }
}

}  // namespace moe
