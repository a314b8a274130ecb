// Load-time weight repack into the tiled gfx950 layout (untimed; the Muse Spark experiment's
// prepare step, and for GPT-OSS checkpoints the gate/up de-interleave and the zero-padding of
// the intermediate dimension described in the "sglang PR 28231" summary).
//
// Prepared buffer, each section 256-byte aligned:
//   codes   [E][N/16][K/64] tiles of 512 bytes; lane l's 8 bytes = dword i (i = 0, 1) holding the
//           eight codes of row l%16 at k = 32 i + 8 (l/16) + 0..7, low nibble = even k
//   scales  NVFP4: [E][N/16][K/64][16 rows][4 e4m3]   (the four groups of 16 of the tile)
//           MXFP4: [E][N/16][K/64][16 rows][2 E8M0]   (the two groups of 32)
//           int4:  [E][N/16][K/128][16 rows] bf16      (one group of 128 per tile pair)
//           asymmetric int4: [E][N/16][K/128][16 rows] u32 = bf16 scale | zero point << 16
//   gs      fp32 [E]                 (NVFP4)
//   bias    bf16 [E][N]              (optional)
// Output row n of a gate/up pair: gate j = n for n < I_pad, up j = n - I_pad otherwise; source
// row j (contiguous halves) or 2j / 2j+1 (interleaved).  Rows j >= I and columns k >= K are
// padding: zero codes, unit scales, zero bias.
#include "moe_internal.h"

namespace moe {

struct PrepGeom {
  int q, E, N, K, Nout, Kout, I, Ip;
  uint32_t flags;
};

// source row of output row n, or -1 for a padding row
__device__ __forceinline__ int src_row(const PrepGeom& g, int n) {
  if (!(g.flags & MOE_PREP_GATE_UP)) return n;
  const int half = n >= g.Ip, j = n - half * g.Ip;
  if (j >= g.I) return -1;
  return (g.flags & MOE_PREP_INTERLEAVED) ? 2 * j + half : half * g.I + j;
}

// Act-order: the stable sort of each expert's input columns by group (g_idx), i.e. prepared
// column j of expert e is input column perm[e][j].  One workgroup per expert: the grouping is
// staged in LDS, then thread t walks the columns in order and places those of group t (and
// t + 256, ...) at group * 128 + rank.  Every group is expected to hold 128 columns; columns
// with an out-of-range group and places beyond 128 per group are skipped, so a bad grouping
// gives wrong (never out-of-bounds) results.
__global__ __launch_bounds__(256) void prep_perm_kernel(const int32_t* __restrict__ g_idx,
                                                        int32_t* __restrict__ perm, int K) {
  __shared__ int32_t s_g[kMaxActOrderK];
  const int e = blockIdx.x, G = K / 128;
  const int32_t* gi = g_idx + (int64_t)e * K;
  int32_t* pe = perm + (int64_t)e * K;
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    s_g[k] = gi[k];
    pe[k] = 0;  // any unfilled place reads column 0 (in bounds)
  }
  __syncthreads();
  for (int grp = threadIdx.x; grp < G; grp += blockDim.x) {
    int cnt = 0;
    for (int k = 0; k < K && cnt < 128; ++k)
      if (s_g[k] == grp) pe[grp * 128 + cnt++] = k;
  }
}

// one thread per output dword of codes
__global__ void prep_codes_kernel(const uint8_t* __restrict__ src, uint32_t* __restrict__ dst, PrepGeom g,
                                  const int32_t* __restrict__ perm) {
  const int NT = g.Nout / kTileN, KT = g.Kout / kTileK;
  const int64_t total = (int64_t)g.E * NT * KT * 128;
  const uint32_t zero = g.q == MOE_Q_INT4_G128 ? 0x88888888u : 0u;
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total;
       d += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(d & 1), lane = (int)((d >> 1) & 63);
    const int64_t tile = d >> 7;
    const int kt = (int)(tile % KT);
    const int64_t et = tile / KT;
    const int nt = (int)(et % NT), e = (int)(et / NT);
    const int n = nt * kTileN + (lane & 15);
    const int k = kt * kTileK + 32 * i + 8 * (lane >> 4);
    const int r = src_row(g, n);
    uint32_t v = zero;
    if (r >= 0 && k < g.K) {
      const uint8_t* p = src + ((int64_t)e * g.N + r) * (g.K / 2);
      if (perm) {  // act-order: gather the eight codes of prepared columns k .. k+7
        const int32_t* pc = perm + (int64_t)e * g.K + k;
        v = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = min(max(pc[j], 0), g.K - 1);
          const uint32_t b = p[c >> 1];
          v |= ((c & 1) ? (b >> 4) : (b & 0xFu)) << (4 * j);
        }
      } else {
        p += k / 2;
        v = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
      }
    }
    dst[d] = v;
  }
}

// one thread per output scale element
__global__ void prep_scales_kernel(const uint8_t* __restrict__ src, const void* __restrict__ zeros,
                                   uint8_t* __restrict__ dst, PrepGeom g) {
  const int NT = g.Nout / kTileN, KT = g.Kout / kTileK;
  const int grp = group_of(g.q);
  const int ngroups = g.K / grp;  // groups per source row
  if (has_zero_points(g.q)) {  // padding: unit scale, zero point 0 (padding codes are 0)
    const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src);
    uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
    const int64_t total = (int64_t)g.E * NT * (KT / 2) * 16;
    for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total;
         d += (int64_t)gridDim.x * blockDim.x) {
      const int row = (int)(d & 15);
      const int64_t t = d >> 4;
      const int kp = (int)(t % (KT / 2));
      const int64_t et = t / (KT / 2);
      const int nt = (int)(et % NT), e = (int)(et / NT);
      const int r = src_row(g, nt * kTileN + row);
      uint32_t v = 0x3F80u;
      if (r >= 0 && kp < ngroups) {
        const int64_t i = ((int64_t)e * g.N + r) * ngroups + kp;
        const uint32_t z = g.q == MOE_Q_INT4ZP_G128 ? (uint32_t)(static_cast<const uint8_t*>(zeros)[i] & 0xF)
                                                    : (uint32_t)static_cast<const uint16_t*>(zeros)[i];
        v = (uint32_t)s16[i] | (z << 16);
      }
      d32[d] = v;
    }
    return;
  }
  if (g.q == MOE_Q_INT4_G128) {
    const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src);
    uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
    const int64_t total = (int64_t)g.E * NT * (KT / 2) * 16;
    for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total;
         d += (int64_t)gridDim.x * blockDim.x) {
      const int row = (int)(d & 15);
      const int64_t t = d >> 4;
      const int kp = (int)(t % (KT / 2));
      const int64_t et = t / (KT / 2);
      const int nt = (int)(et % NT), e = (int)(et / NT);
      const int r = src_row(g, nt * kTileN + row);
      d16[d] = (r >= 0 && kp < ngroups) ? s16[((int64_t)e * g.N + r) * ngroups + kp] : (uint16_t)0x3F80;
    }
    return;
  }
  const int per_row = kTileK / grp;  // 4 (NVFP4) or 2 (MXFP4)
  const uint8_t unit = g.q == MOE_Q_NVFP4_G16 ? 0x38 : 127;  // 1.0 in e4m3fn / E8M0
  const int64_t total = (int64_t)g.E * NT * KT * 16 * per_row;
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total;
       d += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(d % per_row);
    const int64_t t = d / per_row;
    const int row = (int)(t & 15);
    const int64_t tile = t >> 4;
    const int kt = (int)(tile % KT);
    const int64_t et = tile / KT;
    const int nt = (int)(et % NT), e = (int)(et / NT);
    const int r = src_row(g, nt * kTileN + row);
    const int gi = kt * per_row + j;
    dst[d] = (r >= 0 && gi < ngroups) ? src[((int64_t)e * g.N + r) * ngroups + gi] : unit;
  }
}

__global__ void prep_bias_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, PrepGeom g) {
  const int64_t total = (int64_t)g.E * g.Nout;
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total;
       d += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(d % g.Nout), e = (int)(d / g.Nout);
    const int r = src_row(g, n);
    dst[d] = r >= 0 ? src[(int64_t)e * g.N + r] : (uint16_t)0;
  }
}

static int grid_for(int64_t n) { return (int)std::min<int64_t>((n + 255) / 256, 16384); }

// Act-order gather with the source row staged in LDS (K <= kPermLdsK): one wave per row, the
// row read with coalesced 16-byte loads, then each lane gathers its 8 columns from LDS and
// stores 16 bytes.  Rows of dead slots are skipped.
constexpr int kPermLdsK = 4096;
__global__ __launch_bounds__(256) void permute_cols_lds_kernel(
    const uint16_t* __restrict__ src, int64_t ld_src, int row_div, const int32_t* __restrict__ perm,
    int K, int E, const int32_t* __restrict__ slot_expert, int64_t rows, uint16_t* __restrict__ dst,
    int64_t ld_dst) {
  __shared__ __attribute__((aligned(16))) uint16_t s_row[4][kPermLdsK];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint16_t* sr = s_row[w];
  constexpr int J = kPermLdsK / 512;      // 8-column chunks per lane
  for (int64_t r = (int64_t)blockIdx.x * 4 + w; r < rows; r += (int64_t)gridDim.x * 4) {
    const int e = slot_expert[r];          // wave-uniform
    if (e < 0 || e >= E) continue;
    // the lane's column order first (16-byte loads), in flight together with the row's load
    const int32_t* pe = perm + (int64_t)e * K;
    uint4 pv[J][2];
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      const int j = lane * 8 + jj * 512;
      if (j < K) {
        pv[jj][0] = *reinterpret_cast<const uint4*>(pe + j);
        pv[jj][1] = *reinterpret_cast<const uint4*>(pe + j + 4);
      }
    }
    const uint16_t* s = src + (r / row_div) * ld_src;
    for (int c = lane * 8; c < K; c += 512)
      *reinterpret_cast<uint4*>(sr + c) = *reinterpret_cast<const uint4*>(s + c);
    __builtin_amdgcn_s_waitcnt(0xc07f);    // this wave's LDS writes are done (lgkmcnt(0))
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      const int j = lane * 8 + jj * 512;
      if (j < K) {
        const int c[8] = {(int)pv[jj][0].x, (int)pv[jj][0].y, (int)pv[jj][0].z, (int)pv[jj][0].w,
                          (int)pv[jj][1].x, (int)pv[jj][1].y, (int)pv[jj][1].z, (int)pv[jj][1].w};
        uint32_t wv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c0 = min(max(c[2 * i], 0), K - 1), c1 = min(max(c[2 * i + 1], 0), K - 1);
          wv[i] = (uint32_t)sr[c0] | ((uint32_t)sr[c1] << 16);
        }
        *reinterpret_cast<uint4*>(dst + r * ld_dst + j) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    }
    __builtin_amdgcn_wave_barrier();       // every lane's LDS reads before the next row's writes
  }
}

// Act-order gather, any K: one thread per (row, 8 columns); rows of dead slots are skipped.
__global__ void permute_cols_kernel(const uint16_t* __restrict__ src, int64_t ld_src, int row_div,
                                    const int32_t* __restrict__ perm, int K, int E,
                                    const int32_t* __restrict__ slot_expert, int64_t rows,
                                    uint16_t* __restrict__ dst, int64_t ld_dst) {
  const int chunks = K >> 3;
  const int64_t total = rows * chunks;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / chunks;
    const int j = (int)(t - r * chunks) << 3;
    const int e = slot_expert[r];
    if (e < 0 || e >= E) continue;
    const uint16_t* s = src + (r / row_div) * ld_src;
    const int32_t* pc = perm + (int64_t)e * K + j;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c0 = min(max(pc[2 * i], 0), K - 1), c1 = min(max(pc[2 * i + 1], 0), K - 1);
      w[i] = (uint32_t)s[c0] | ((uint32_t)s[c1] << 16);
    }
    *reinterpret_cast<uint4*>(dst + r * ld_dst + j) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_permute_cols(const uint16_t* src, int64_t ld_src, int32_t row_div, const int32_t* perm,
                                int32_t K, int32_t E, const int32_t* slot_expert, int64_t rows, uint16_t* dst,
                                int64_t ld_dst, hipStream_t stream) {
  MOE_REQUIRE(rows >= 0 && K >= 8 && K % 8 == 0 && E >= 1 && row_div >= 1, MOE_EINVAL,
              "moe_permute_cols: rows=%lld K=%d E=%d row_div=%d", (long long)rows, K, E, row_div);
  MOE_REQUIRE(ld_src >= K && ld_dst >= K && ld_dst % 8 == 0, MOE_EINVAL,
              "moe_permute_cols: ld_src=%lld ld_dst=%lld (>= K, ld_dst a multiple of 8)",
              (long long)ld_src, (long long)ld_dst);
  if (rows == 0) return ok();
  MOE_REQUIRE(src && perm && slot_expert && dst, MOE_EINVAL, "moe_permute_cols: null pointer");
  MOE_REQUIRE(((uintptr_t)dst & 15) == 0, MOE_EINVAL, "moe_permute_cols: dst must be 16-byte aligned");
  if (K <= kPermLdsK && ((uintptr_t)src & 15) == 0 && ld_src % 8 == 0) {
    const int grid = (int)std::min<int64_t>((rows + 3) / 4, 16384);
    hipLaunchKernelGGL(permute_cols_lds_kernel, dim3(grid), dim3(256), 0, stream, src, ld_src, (int)row_div,
                       perm, (int)K, (int)E, slot_expert, rows, dst, ld_dst);
    return check_launch("moe_permute_cols");
  }
  const int64_t total = rows * (K / 8);
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 16384);
  hipLaunchKernelGGL(permute_cols_kernel, dim3(grid), dim3(256), 0, stream, src, ld_src, (int)row_div, perm,
                     (int)K, (int)E, slot_expert, rows, dst, ld_dst);
  return check_launch("moe_permute_cols");
}

extern "C" int moe_w4a16_prepare(moe_qtype q, const uint8_t* codes, const void* scales,
                                 const float* global_scale, const uint16_t* bias, const void* zeros,
                                 const int32_t* g_idx, int32_t E, int32_t N, int32_t K, uint32_t flags,
                                 void* out, size_t out_bytes, moe_weights* desc, hipStream_t stream) {
  int32_t Nout = 0, Kout = 0;
  size_t need = 0;
  int rc = moe_w4a16_prepared_size(q, E, N, K, flags, bias != nullptr, &Nout, &Kout, &need);
  if (rc) return rc;
  MOE_REQUIRE(codes && scales && out && desc, MOE_EINVAL, "moe_w4a16_prepare: null pointer");
  MOE_REQUIRE((q == MOE_Q_NVFP4_G16) == (global_scale != nullptr), MOE_EINVAL,
              "moe_w4a16_prepare: a global scale is required for NVFP4 and only for NVFP4");
  MOE_REQUIRE(has_zero_points(q) == (zeros != nullptr), MOE_EINVAL,
              "moe_w4a16_prepare: zero points are required for asymmetric int4 and only for it");
  MOE_REQUIRE(((flags & MOE_PREP_ACT_ORDER) != 0) == (g_idx != nullptr), MOE_EINVAL,
              "moe_w4a16_prepare: g_idx is required with MOE_PREP_ACT_ORDER and only with it");
  MOE_REQUIRE(out_bytes >= need, MOE_ESIZE, "moe_w4a16_prepare: out has %zu bytes, %zu needed",
              out_bytes, need);
  MOE_REQUIRE(((uintptr_t)out & 255) == 0, MOE_EINVAL, "moe_w4a16_prepare: out must be 256-byte aligned");
  PrepGeom g{(int)q, E, N, K, Nout, Kout, (flags & MOE_PREP_GATE_UP) ? N / 2 : N,
             (flags & MOE_PREP_GATE_UP) ? Nout / 2 : Nout, flags};
  const size_t tiles = (size_t)E * (Nout / kTileN) * (Kout / kTileK);
  uint8_t* base = static_cast<uint8_t*>(out);
  uint8_t* p_codes = base;
  uint8_t* p_scales = p_codes + align256(tiles * kTileBytes);
  uint8_t* p_gs = p_scales + align256(tiles * (size_t)scale_bytes_per_tile(q));
  uint8_t* p_bias = p_gs + (q == MOE_Q_NVFP4_G16 ? align256((size_t)E * 4) : 0);
  int32_t* p_perm = reinterpret_cast<int32_t*>(p_bias + (bias ? align256((size_t)E * Nout * 2) : 0));

  if (g_idx)
    hipLaunchKernelGGL(prep_perm_kernel, dim3(E), dim3(256), 0, stream, g_idx, p_perm, K);
  hipLaunchKernelGGL(prep_codes_kernel, dim3(grid_for((int64_t)tiles * 128)), dim3(256), 0, stream,
                     codes, reinterpret_cast<uint32_t*>(p_codes), g, g_idx ? p_perm : nullptr);
  hipLaunchKernelGGL(prep_scales_kernel, dim3(grid_for((int64_t)tiles * 64)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(scales), zeros, p_scales, g);
  if (q == MOE_Q_NVFP4_G16) {
    hipError_t e = hipMemcpyAsync(p_gs, global_scale, (size_t)E * 4, hipMemcpyDeviceToDevice, stream);
    MOE_REQUIRE(e == hipSuccess, MOE_EHIP, "moe_w4a16_prepare: copy of the global scales: %s",
                hipGetErrorString(e));
  }
  if (bias)
    hipLaunchKernelGGL(prep_bias_kernel, dim3(grid_for((int64_t)E * Nout)), dim3(256), 0, stream,
                       bias, reinterpret_cast<uint16_t*>(p_bias), g);
  rc = check_launch("moe_w4a16_prepare");
  if (rc) return rc;
  moe_weights d{};
  d.qtype = q;
  d.n_experts = E;
  d.N = Nout;
  d.K = Kout;
  d.N_logical = N;
  d.K_logical = K;
  d.flags = flags;
  d.codes = p_codes;
  d.scales = p_scales;
  d.global_scale = q == MOE_Q_NVFP4_G16 ? reinterpret_cast<const float*>(p_gs) : nullptr;
  d.bias = bias ? reinterpret_cast<const uint16_t*>(p_bias) : nullptr;
  d.perm = g_idx ? p_perm : nullptr;
  *desc = d;
  return ok();
}
