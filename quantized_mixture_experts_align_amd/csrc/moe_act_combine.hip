// Gated activation and the top-k weighted combine (with the optional post-expert RMSNorm),
// plus the norm-weight binding bf16(1 + w).
//
// Both kernels stream bf16 rows with 16-byte loads (8 values per lane) and compute in fp32.
#include <algorithm>
#include <cmath>

#include "moe_internal.h"

namespace moe {

// One thread per 8 output columns of one row; grid-stride over rows x chunks.
template <class Act>
__global__ __launch_bounds__(256) void act_kernel(const uint16_t* __restrict__ in, int32_t ld_in,
                                                  uint16_t* __restrict__ out, int32_t ld_out,
                                                  int64_t R, int32_t I,
                                                  const int32_t* __restrict__ slot_local, Act act) {
  const int chunks = I >> 3;
  const int64_t total = R * chunks;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = c / chunks;
    const int col = (int)(c - r * chunks) << 3;
    if (slot_local && slot_local[r] < 0) continue;
    const uint4 g = *reinterpret_cast<const uint4*>(in + r * ld_in + col);
    const uint4 u = *reinterpret_cast<const uint4*>(in + r * ld_in + I + col);
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = pack_bf16x2(act(bf16_lo(gw[j]), bf16_lo(uw[j])), act(bf16_hi(gw[j]), bf16_hi(uw[j])));
    *reinterpret_cast<uint4*>(out + r * ld_out + col) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Non-gated activation: one thread per 8 columns of one row, out = act(in) element-wise.
template <class Act>
__global__ __launch_bounds__(256) void act1_kernel(const uint16_t* __restrict__ in, int32_t ld_in,
                                                   uint16_t* __restrict__ out, int32_t ld_out, int64_t R,
                                                   int32_t I, const int32_t* __restrict__ slot_local, Act act) {
  const int chunks = I >> 3;
  const int64_t total = R * chunks;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = c / chunks;
    const int col = (int)(c - r * chunks) << 3;
    if (slot_local && slot_local[r] < 0) continue;
    const uint4 h = *reinterpret_cast<const uint4*>(in + r * ld_in + col);
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(act(bf16_lo(hw[j])), act(bf16_hi(hw[j])));
    *reinterpret_cast<uint4*>(out + r * ld_out + col) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

constexpr int kCombineThreads = 256;
constexpr int kMaxTopK = 16;

// One workgroup per token.  With a norm: pass 1 reduces sum((y * nw)^2) per live slot, pass 2
// forms sum_s g_s / sqrt(ss_s / H + eps) * y_s * nw.  Dead slots are never read.
template <bool NORM>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const uint16_t* __restrict__ y, const float* __restrict__ gw, const int32_t* __restrict__ slot_local,
    const uint16_t* __restrict__ nw, float eps, float rsf, int32_t top_k, int32_t H, uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __shared__ float fac[kMaxTopK];
  __shared__ float red[kCombineThreads / 64][kMaxTopK];
  uint32_t live = 0;
  for (int s = 0; s < top_k; ++s)
    if (slot_local[t * top_k + s] >= 0) live |= 1u << s;
  const int chunks = H >> 3;
  if (NORM) {
    float ss[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) ss[s] = 0.f;
    for (int c = tid; c < chunks; c += kCombineThreads) {
      const uint4 nv = *reinterpret_cast<const uint4*>(nw + c * 8);
      const uint32_t n4[4] = {nv.x, nv.y, nv.z, nv.w};
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s) {
        if (s >= top_k || !((live >> s) & 1)) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(y + ((t * top_k + s) * (int64_t)H) + c * 8);
        const uint32_t v4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = bf16_lo(v4[j]) * bf16_lo(n4[j]), b = bf16_hi(v4[j]) * bf16_hi(n4[j]);
          ss[s] = fmaf(a, a, ss[s]);
          ss[s] = fmaf(b, b, ss[s]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
      if (s >= top_k) break;
      float v = ss[s];
      for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
      if (lane == 0) red[w][s] = v;
    }
    __syncthreads();
    if (tid < top_k) {
      float v = 0.f;
      for (int i = 0; i < kCombineThreads / 64; ++i) v += red[i][tid];
      const float g = gw[t * top_k + tid];
      fac[tid] = ((live >> tid) & 1) ? g / sqrtf(v / (float)H + eps) : 0.f;
    }
    __syncthreads();
  }
  for (int c = tid; c < chunks; c += kCombineThreads) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    uint32_t n4[4] = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    if (NORM) {
      const uint4 nv = *reinterpret_cast<const uint4*>(nw + c * 8);
      n4[0] = nv.x; n4[1] = nv.y; n4[2] = nv.z; n4[3] = nv.w;
    }
    for (int s = 0; s < top_k; ++s) {
      if (!((live >> s) & 1)) continue;
      const float f = NORM ? fac[s] : gw[t * top_k + s];
      const uint4 v = *reinterpret_cast<const uint4*>(y + ((t * top_k + s) * (int64_t)H) + c * 8);
      const uint32_t v4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (NORM) {
          acc[2 * j] = fmaf(f, bf16_lo(v4[j]) * bf16_lo(n4[j]), acc[2 * j]);
          acc[2 * j + 1] = fmaf(f, bf16_hi(v4[j]) * bf16_hi(n4[j]), acc[2 * j + 1]);
        } else {
          acc[2 * j] = fmaf(f, bf16_lo(v4[j]), acc[2 * j]);
          acc[2 * j + 1] = fmaf(f, bf16_hi(v4[j]), acc[2 * j + 1]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= rsf;  // routed scaling factor (1 = none)
    *reinterpret_cast<uint4*>(out + t * H + c * 8) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

// Single pass for top_k <= TK and rows of at most CP * blockDim.x chunks of 8 columns.  Every
// operand of the token is requested up front -- slot flags, weights, norm weight and the slots'
// y chunks (with `spec`, also the chunks of slots that may be dead, so that nothing waits for
// the flags; their values are never used) -- so a token costs one round trip to memory, and y
// stays in registers between the norm's reduction and the weighted sum (read once).  The fp32
// operations and their order per output are those of combine_kernel.
template <bool NORM, int TK, int CP>
__global__ __launch_bounds__(512) void combine1_kernel(
    const uint16_t* __restrict__ y, const float* __restrict__ gw, const int32_t* __restrict__ slot_local,
    const uint16_t* __restrict__ nw, float eps, float rsf, int32_t top_k, int32_t H, int32_t spec,
    uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, T = blockDim.x;
  __shared__ float red[8][TK];
  __shared__ float fac[TK], gl[TK];
  const int chunks = H >> 3;
  uint32_t live = 0;
  float g[TK];
#pragma unroll
  for (int s = 0; s < TK; ++s) {
    g[s] = 0.f;
    if (s < top_k) {
      g[s] = gw[t * top_k + s];
      if (slot_local[t * top_k + s] >= 0) live |= 1u << s;
    }
  }
  uint4 v[TK][CP], nv[CP];
#pragma unroll
  for (int c = 0; c < CP; ++c) {
    const int col = tid + c * T;
    nv[c] = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    if (NORM && col < chunks) nv[c] = *reinterpret_cast<const uint4*>(nw + col * 8);
#pragma unroll
    for (int s = 0; s < TK; ++s) {
      v[s][c] = make_uint4(0u, 0u, 0u, 0u);
      if (s < top_k && col < chunks && (spec || ((live >> s) & 1)))
        v[s][c] = *reinterpret_cast<const uint4*>(y + (t * top_k + s) * (int64_t)H + col * 8);
    }
  }
  float f[TK];
  if (NORM) {
#pragma unroll
    for (int s = 0; s < TK; ++s) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < CP; ++c) {
        if (tid + c * T >= chunks || !((live >> s) & 1)) continue;
        const uint32_t v4[4] = {v[s][c].x, v[s][c].y, v[s][c].z, v[s][c].w};
        const uint32_t n4[4] = {nv[c].x, nv[c].y, nv[c].z, nv[c].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = bf16_lo(v4[j]) * bf16_lo(n4[j]), b = bf16_hi(v4[j]) * bf16_hi(n4[j]);
          ss = fmaf(a, a, ss);
          ss = fmaf(b, b, ss);
        }
      }
      for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d);
      if (lane == 0 && s < top_k) red[w][s] = ss;
      if (tid == 0) gl[s] = g[s];
    }
    __syncthreads();
    if (tid < top_k) {
      float ssum = 0.f;
      for (int i = 0; i < T / 64; ++i) ssum += red[i][tid];
      fac[tid] = ((live >> tid) & 1) ? gl[tid] / sqrtf(ssum / (float)H + eps) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < TK; ++s) f[s] = s < top_k ? fac[s] : 0.f;
  } else {
#pragma unroll
    for (int s = 0; s < TK; ++s) f[s] = g[s];
  }
#pragma unroll
  for (int c = 0; c < CP; ++c) {
    const int col = tid + c * T;
    if (col >= chunks) break;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    const uint32_t n4[4] = {nv[c].x, nv[c].y, nv[c].z, nv[c].w};
#pragma unroll
    for (int s = 0; s < TK; ++s) {
      if (s >= top_k || !((live >> s) & 1)) continue;
      const uint32_t v4[4] = {v[s][c].x, v[s][c].y, v[s][c].z, v[s][c].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (NORM) {
          acc[2 * j] = fmaf(f[s], bf16_lo(v4[j]) * bf16_lo(n4[j]), acc[2 * j]);
          acc[2 * j + 1] = fmaf(f[s], bf16_hi(v4[j]) * bf16_hi(n4[j]), acc[2 * j + 1]);
        } else {
          acc[2 * j] = fmaf(f[s], bf16_lo(v4[j]), acc[2 * j]);
          acc[2 * j + 1] = fmaf(f[s], bf16_hi(v4[j]), acc[2 * j + 1]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= rsf;  // routed scaling factor (1 = none)
    *reinterpret_cast<uint4*>(out + t * H + col * 8) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

template <bool NORM, int TK>
static void launch_combine1(int CP, int T, int64_t M, const uint16_t* y, const float* gw, const int32_t* sl,
                            const uint16_t* nw, float eps, float rsf, int top_k, int H, int spec, uint16_t* out,
                            hipStream_t st) {
  if (CP == 1)
    hipLaunchKernelGGL((combine1_kernel<NORM, TK, 1>), dim3((unsigned)M), dim3(T), 0, st, y, gw, sl, nw, eps, rsf, top_k, H, spec, out);
  else
    hipLaunchKernelGGL((combine1_kernel<NORM, TK, 2>), dim3((unsigned)M), dim3(T), 0, st, y, gw, sl, nw, eps, rsf, top_k, H, spec, out);
}

__global__ void norm_weight_kernel(const uint16_t* __restrict__ w, int32_t H, uint16_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < H) out[i] = f32_to_bf16(1.0f + bf16_to_f32(w[i]));
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace moe

using namespace moe;

extern "C" int moe_act(moe_act_kind kind, const uint16_t* in, int32_t ld_in, uint16_t* out,
                       int32_t ld_out, int64_t R, int32_t I, const int32_t* slot_local_ids,
                       float alpha, float limit, hipStream_t stream) {
  MOE_REQUIRE(kind == MOE_ACT_SILU_MUL || kind == MOE_ACT_SWIGLU_ALPHA || kind == MOE_ACT_RELU2, MOE_EINVAL,
              "moe_act: unknown activation %d", (int)kind);
  const bool gated = kind != MOE_ACT_RELU2;
  MOE_REQUIRE(R >= 0 && I >= 1, MOE_EINVAL, "moe_act: R=%lld I=%d", (long long)R, I);
  MOE_REQUIRE(I % 8 == 0 && ld_in % 8 == 0 && ld_out % 8 == 0, MOE_EUNSUPPORTED,
              "moe_act: I, ld_in and ld_out must be multiples of 8 (I=%d ld_in=%d ld_out=%d)", I,
              ld_in, ld_out);
  MOE_REQUIRE(ld_in >= (gated ? 2 * I : I) && ld_out >= I, MOE_EINVAL, "moe_act: leading dims too small");
  if (R == 0) return ok();
  MOE_REQUIRE(in && out, MOE_EINVAL, "moe_act: null pointer");
  MOE_REQUIRE(aligned16(in) && aligned16(out), MOE_EUNSUPPORTED, "moe_act: pointers must be 16-byte aligned");
  const int64_t total = R * (I / 8);
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
  if (kind == MOE_ACT_SILU_MUL)
    hipLaunchKernelGGL(act_kernel<SiluMul>, dim3(blocks), dim3(256), 0, stream, in, ld_in, out,
                       ld_out, R, I, slot_local_ids, SiluMul{alpha, limit});
  else if (kind == MOE_ACT_RELU2)
    hipLaunchKernelGGL(act1_kernel<Relu2>, dim3(blocks), dim3(256), 0, stream, in, ld_in, out,
                       ld_out, R, I, slot_local_ids, Relu2{alpha, limit});
  else
    hipLaunchKernelGGL(act_kernel<SwigluAlpha>, dim3(blocks), dim3(256), 0, stream, in, ld_in, out,
                       ld_out, R, I, slot_local_ids, SwigluAlpha{alpha, limit});
  return check_launch("moe_act");
}

extern "C" int moe_combine(const uint16_t* y, const float* topk_weights, const int32_t* slot_local_ids,
                           const uint16_t* norm_w, float eps, float routed_scaling_factor, int64_t M,
                           int32_t top_k, int32_t H, uint16_t* out, hipStream_t stream) {
  const float rsf = routed_scaling_factor;
  MOE_REQUIRE(M >= 0 && top_k >= 1 && top_k <= kMaxTopK, MOE_EUNSUPPORTED,
              "moe_combine: M=%lld top_k=%d (top_k must be 1..%d)", (long long)M, top_k, kMaxTopK);
  MOE_REQUIRE(H >= 8 && H % 8 == 0, MOE_EUNSUPPORTED, "moe_combine: H=%d must be a multiple of 8", H);
  MOE_REQUIRE(M <= 0x7FFFFFFF, MOE_EUNSUPPORTED, "moe_combine: M too large");
  if (M == 0) return ok();
  MOE_REQUIRE(y && topk_weights && slot_local_ids && out, MOE_EINVAL, "moe_combine: null pointer");
  MOE_REQUIRE(aligned16(y) && aligned16(out) && (!norm_w || aligned16(norm_w)), MOE_EUNSUPPORTED,
              "moe_combine: bf16 tensors must be 16-byte aligned");
  // single pass when a token's slots fit in registers: top_k <= 8, H <= 2 * 512 * 8; one
  // 16-B chunk per thread up to 512 threads (more loads in flight per token)
  const int chunks = H / 8;
  if (top_k <= 8 && chunks <= 1024) {
    const int T = std::min(512, (chunks + 63) / 64 * 64), CP = (chunks + T - 1) / T;
    const int spec = M <= 256;  // small batches: do not wait for the slot flags before reading y
    if (norm_w) {
      if (top_k <= 2) launch_combine1<true, 2>(CP, T, M, y, topk_weights, slot_local_ids, norm_w, eps, rsf, top_k, H, spec, out, stream);
      else if (top_k <= 4) launch_combine1<true, 4>(CP, T, M, y, topk_weights, slot_local_ids, norm_w, eps, rsf, top_k, H, spec, out, stream);
      else launch_combine1<true, 8>(CP, T, M, y, topk_weights, slot_local_ids, norm_w, eps, rsf, top_k, H, spec, out, stream);
    } else {
      if (top_k <= 2) launch_combine1<false, 2>(CP, T, M, y, topk_weights, slot_local_ids, norm_w, eps, rsf, top_k, H, spec, out, stream);
      else if (top_k <= 4) launch_combine1<false, 4>(CP, T, M, y, topk_weights, slot_local_ids, norm_w, eps, rsf, top_k, H, spec, out, stream);
      else launch_combine1<false, 8>(CP, T, M, y, topk_weights, slot_local_ids, norm_w, eps, rsf, top_k, H, spec, out, stream);
    }
    return check_launch("moe_combine");
  }
  if (norm_w)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)M), dim3(kCombineThreads), 0, stream, y,
                       topk_weights, slot_local_ids, norm_w, eps, rsf, top_k, H, out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)M), dim3(kCombineThreads), 0, stream, y,
                       topk_weights, slot_local_ids, norm_w, eps, rsf, top_k, H, out);
  return check_launch("moe_combine");
}

extern "C" int moe_norm_weight(const uint16_t* w, int32_t H, uint16_t* out, hipStream_t stream) {
  MOE_REQUIRE(H >= 1, MOE_EINVAL, "moe_norm_weight: H=%d", H);
  MOE_REQUIRE(w && out, MOE_EINVAL, "moe_norm_weight: null pointer");
  hipLaunchKernelGGL(norm_weight_kernel, dim3((H + 255) / 256), dim3(256), 0, stream, w, H, out);
  return check_launch("moe_norm_weight");
}
