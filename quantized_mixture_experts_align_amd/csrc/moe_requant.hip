// moe_fp8_requant: the W4AFP8 activation requant of the "sglang PR 35760" summary (sections
// "Feature and motivation" and "Implementation breakdown", items 1-3).  After the low-latency
// dispatch, expert e holds max_m row slots of K float8 e4m3fn codes, the first masked_m[e] of
// them live, each quantised with one fp32 scale per 128-wide group of K (per token and group).
// The W4A8 GEMM wants one scale for the whole tensor, so every live element becomes
//
//   code' = e4m3fn_saturating( float32( float32(x * s) * r ) ),   r = float32(1 / tensor_scale),
//
// two multiplies per element and two bytes moved (one read, one written).
//
// Schedule.  The page replaces a fixed grid of programs per expert (most of which only load the
// mask and exit when rows are sparse) by a per-expert row cap plus a second phase in which the
// rows above the cap are found through a prefix sum over the row counts and shared by the whole
// launch.  Here every row takes that second path: each wave scans masked_m itself (up to 1024
// experts, 16 per lane, held in registers), so the live rows form one flat index space of
// sum(masked_m) rows x ceil(K / 1024) chunks.  A work item is one 1024-byte chunk of one live row
// -- 16 bytes per lane, one 128-bit load and one 128-bit store -- and the waves of a grid sized
// to the machine take items round-robin, several loads in flight per lane.  No program is ever
// spent on a dead row slot, and a hot expert's rows spread over every CU like anyone else's
// (the skew the page's overflow phase exists for), with no row-count estimate from the host.
// Each lane maps its item to (expert, row) with one ballot over the lanes' prefix sums and a
// short search inside the owning lane's 16 counts.  Every output byte depends only on its own
// input byte and group scale, so results are the same for every grid and unroll.
//
// Scales are addressed through element strides (e, row, group), so the row-major
// [E, max_m, K/group] layout and DeepEP's column-major one ([E, K/group, max_m] per expert) are
// the same code; a lane loads its group's scale once (the eight lanes of a group share the
// address), never one gather per element as in the layout the page starts from.
#include <algorithm>
#include <cmath>

#include "moe_internal.h"

namespace moe {

int device_cu_count();

constexpr int kRqWaves = 4;          // waves per workgroup
constexpr int kRqChunk = 64 * 16;    // bytes of one work item: 64 lanes x 16 bytes
constexpr int kRqMaxExperts = 1024;  // 64 lanes x 16 counts
constexpr float kE4m3Max = 448.0f;

// Four float32 values -> four float8 e4m3fn codes (byte i = value i), saturating: magnitudes are
// clamped to 448 before the hardware's round-to-nearest-even conversion (gfx950 converts to the
// OCP e4m3 format; unclamped, it sends everything above 464 to NaN), the sign is kept (so
// -0 -> 0x80), and NaN gives 0x7F.  The general path, for any scale.
__device__ __forceinline__ uint32_t encode4_e4m3_sat(float v0, float v1, float v2, float v3) {
  const float c0 = copysignf(fminf(fabsf(v0), kE4m3Max), v0);
  const float c1 = copysignf(fminf(fabsf(v1), kE4m3Max), v1);
  const float c2 = copysignf(fminf(fabsf(v2), kE4m3Max), v2);
  const float c3 = copysignf(fminf(fabsf(v3), kE4m3Max), v3);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, (int)w, true);
  const uint32_t nan = (v0 != v0 ? 0x000000FFu : 0u) | (v1 != v1 ? 0x0000FF00u : 0u) |
                       (v2 != v2 ? 0x00FF0000u : 0u) | (v3 != v3 ? 0xFF000000u : 0u);
  return (w & ~nan) | (0x7F7F7F7Fu & nan);
}

// Four codes of one dword requantised with the (x * s) * r of the page, in that order; any s, r.
__device__ __forceinline__ uint32_t requant4(uint32_t d, float s, float r) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)d, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)d, true);
  return encode4_e4m3_sat((lo[0] * s) * r, (lo[1] * s) * r, (hi[0] * s) * r, (hi[1] * s) * r);
}

// The same for a finite s and a finite, non-zero r.  Then (x * s) * r is NaN exactly when the
// code x is (0x7F / 0xFF): a finite product can overflow to +-inf, but inf times a finite non-zero
// r stays inf.  med3(v, -448, 448) equals the clamp above for every value but NaN (checked on
// the device over all 2^32 float32 inputs), and the NaN outputs are set from the input codes with
// byte-wise integer arithmetic: a byte whose low seven bits are all ones is NaN.
__device__ __forceinline__ uint32_t requant4_finite(uint32_t d, float s, float r) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)d, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)d, true);
  const float c0 = __builtin_amdgcn_fmed3f((lo[0] * s) * r, -kE4m3Max, kE4m3Max);
  const float c1 = __builtin_amdgcn_fmed3f((lo[1] * s) * r, -kE4m3Max, kE4m3Max);
  const float c2 = __builtin_amdgcn_fmed3f((hi[0] * s) * r, -kE4m3Max, kE4m3Max);
  const float c3 = __builtin_amdgcn_fmed3f((hi[1] * s) * r, -kE4m3Max, kE4m3Max);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, (int)w, true);
  const uint32_t h = ((d & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;  // bit 7 set: NaN byte
  const uint32_t m = (h - (h >> 7)) | h;                                 // 0x80 -> 0xFF
  return (w & ~m) | (0x7F7F7F7Fu & m);
}

// PMAX = counts per lane (experts <= 64 * PMAX), U = items in flight per wave.
template <int PMAX, int U>
__global__ __launch_bounds__(kRqWaves * 64) void requant_kernel(
    const uint8_t* x, uint8_t* out, const float* __restrict__ scales, int64_t sse,  // out may be x
    int64_t ssm, int64_t ssg, const int32_t* __restrict__ masked_m,
    const float* __restrict__ tensor_scale, int E, int max_m, int K, int group, int chunks) {
  const int lane = threadIdx.x & 63;
  // Row counts of this lane's experts [lane*PMAX, lane*PMAX + PMAX), clamped to [0, max_m], and
  // their running sums inside the lane; then the lanes' exclusive offsets by a wave scan.
  int incl[PMAX];
  int tot = 0;
#pragma unroll
  for (int p = 0; p < PMAX; ++p) {
    const int e = lane * PMAX + p;
    const int c = e < E ? min(max(masked_m[e], 0), max_m) : 0;
    tot += c;
    incl[p] = tot;
  }
  int scan = tot;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(scan, d);
    if (lane >= d) scan += o;
  }
  const int excl = scan - tot;
  const int rows = __shfl(scan, 63);                  // live rows in the batch
  const int items = rows * chunks;                    // < 2^31, checked on the host
  const float r = 1.0f / *tensor_scale;               // correctly rounded fp32 division
  const bool r_finite = __builtin_isfinite(r) && r != 0.0f;
  const int waves = gridDim.x * kRqWaves;
  const int first = blockIdx.x * kRqWaves + (threadIdx.x >> 6);

  for (int base = first; base < items; base += waves * U) {
    uint4 v[U];
    float s[U];
    int64_t off[U];
    bool go[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * waves;                 // wave-uniform
      go[u] = false;
      v[u] = make_uint4(0, 0, 0, 0);
      s[u] = 0.0f;
      off[u] = 0;
      if (i < items) {
        const int row = i / chunks;                   // flat live-row index
        const int kb = (i - row * chunks) * kRqChunk + lane * 16;
        // owner lane: the last lane whose offset is <= row (offsets never decrease)
        const int j = __popcll(__ballot(excl <= row)) - 1;
        // inside every lane, the number of its experts that end at or before the row, and
        // where the next one starts; only lane j's answer is used
        const int rr = row - excl;
        int el = 0, start = 0;
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
          if (incl[p] <= rr) {
            ++el;
            start = incl[p];
          }
        }
        const int e = __shfl(lane * PMAX + el, j);
        const int m = row - __shfl(excl + start, j);
        if (kb < K) {
          go[u] = true;
          off[u] = ((int64_t)e * max_m + m) * K + kb;
          v[u] = *reinterpret_cast<const uint4*>(x + off[u]);
          s[u] = scales[(int64_t)e * sse + (int64_t)m * ssm + (int64_t)(kb / group) * ssg];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (go[u]) {
        uint4 o;
        if (__builtin_isfinite(s[u]) && r_finite) {
          o.x = requant4_finite(v[u].x, s[u], r);
          o.y = requant4_finite(v[u].y, s[u], r);
          o.z = requant4_finite(v[u].z, s[u], r);
          o.w = requant4_finite(v[u].w, s[u], r);
        } else {
          o.x = requant4(v[u].x, s[u], r);
          o.y = requant4(v[u].y, s[u], r);
          o.z = requant4(v[u].z, s[u], r);
          o.w = requant4(v[u].w, s[u], r);
        }
        *reinterpret_cast<uint4*>(out + off[u]) = o;
      }
    }
  }
}

template <int PMAX>
static void launch_pmax(int unroll, int grid, hipStream_t st, const uint8_t* x, uint8_t* out,
                        const float* scales, int64_t sse, int64_t ssm, int64_t ssg,
                        const int32_t* masked_m, const float* ts, int E, int max_m, int K, int group,
                        int chunks) {
  const dim3 g(grid), b(kRqWaves * 64);
  switch (unroll) {
    case 1:
      requant_kernel<PMAX, 1><<<g, b, 0, st>>>(x, out, scales, sse, ssm, ssg, masked_m, ts, E, max_m, K, group, chunks);
      break;
    case 2:
      requant_kernel<PMAX, 2><<<g, b, 0, st>>>(x, out, scales, sse, ssm, ssg, masked_m, ts, E, max_m, K, group, chunks);
      break;
    default:
      requant_kernel<PMAX, 4><<<g, b, 0, st>>>(x, out, scales, sse, ssm, ssg, masked_m, ts, E, max_m, K, group, chunks);
      break;
  }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_fp8_requant_choose(int32_t E, int32_t max_m, int32_t K, int32_t expected_rows,
                                      int32_t num_cus, moe_requant_config* cfg) {
  MOE_REQUIRE(cfg, MOE_EINVAL, "moe_fp8_requant_choose: null config");
  MOE_REQUIRE(E >= 0 && max_m >= 0 && K >= 16 && num_cus >= 1, MOE_EINVAL,
              "moe_fp8_requant_choose: E=%d max_m=%d K=%d num_cus=%d out of range", E, max_m, K,
              num_cus);
  // Work items if every expert has expected_rows live rows (all row slots when unknown), and the
  // most the batch can have.  About two items per wave (measured: fewer waves leave the stream
  // latency-bound, more pay the per-wave scan for nothing), as 2, 4 or 8 workgroups of four
  // waves per CU, never more waves than possible items; beyond eight workgroups per CU a wave
  // takes two or four items at a time.
  const int64_t chunks = (K + kRqChunk - 1) / kRqChunk;
  const int64_t rows = expected_rows > 0 ? std::min(expected_rows, max_m) : max_m;
  const int64_t items = std::max<int64_t>(1, (int64_t)E * rows * chunks);
  const int64_t max_items = std::max<int64_t>(1, (int64_t)E * max_m * chunks);
  const int64_t want = (items + 2 * kRqWaves - 1) / (2 * kRqWaves);
  // 2, 4 or 8 workgroups on every CU (measured: 924 -> 1024 and 1792 -> 2048 workgroups are
  // 5-12% faster on 256 CUs)
  int64_t wg = 2 * (int64_t)num_cus;
  while (wg < want && wg < 8 * (int64_t)num_cus) wg *= 2;
  wg = std::max<int64_t>(1, std::min(wg, (max_items + kRqWaves - 1) / kRqWaves));
  cfg->workgroups = (int32_t)wg;
  const int64_t per_wave = (items + wg * kRqWaves - 1) / (wg * kRqWaves);
  cfg->unroll = per_wave > 4 ? 4 : (per_wave > 2 ? 2 : 1);
  return ok();
}

extern "C" int moe_fp8_requant(const uint8_t* x, const float* scales, int64_t scale_stride_e,
                               int64_t scale_stride_m, int64_t scale_stride_g,
                               const int32_t* masked_m, const float* tensor_scale, int32_t E,
                               int32_t max_m, int32_t K, int32_t group_size, uint8_t* out,
                               const moe_requant_config* cfg, hipStream_t stream) {
  MOE_REQUIRE(E >= 0 && max_m >= 0, MOE_EINVAL, "moe_fp8_requant: E=%d max_m=%d must be >= 0", E,
              max_m);
  MOE_REQUIRE(E <= kRqMaxExperts, MOE_EUNSUPPORTED, "moe_fp8_requant: E=%d above %d experts", E,
              kRqMaxExperts);
  MOE_REQUIRE(group_size >= 16 && group_size % 16 == 0, MOE_EUNSUPPORTED,
              "moe_fp8_requant: group_size=%d must be a positive multiple of 16", group_size);
  MOE_REQUIRE(K >= group_size && K % group_size == 0, MOE_EINVAL,
              "moe_fp8_requant: K=%d is not a positive multiple of group_size=%d", K, group_size);
  const int64_t chunks = (K + kRqChunk - 1) / kRqChunk;
  MOE_REQUIRE((int64_t)E * max_m * chunks < ((int64_t)1 << 31) &&
                  (int64_t)E * max_m < ((int64_t)1 << 31),
              MOE_EUNSUPPORTED, "moe_fp8_requant: %d x %d rows of K=%d exceed 2^31 work items", E,
              max_m, K);
  if (E == 0 || max_m == 0) return ok();  // no row slots: nothing to launch
  MOE_REQUIRE(x && scales && masked_m && tensor_scale && out, MOE_EINVAL,
              "moe_fp8_requant: null device pointer");
  MOE_REQUIRE(((uintptr_t)x & 15) == 0 && ((uintptr_t)out & 15) == 0 && K % 16 == 0, MOE_EINVAL,
              "moe_fp8_requant: x and out must be 16-byte aligned");
  MOE_REQUIRE(scale_stride_e >= 0 && scale_stride_m >= 0 && scale_stride_g >= 0, MOE_EINVAL,
              "moe_fp8_requant: negative scale stride");
  MOE_REQUIRE(out == x || out + (int64_t)E * max_m * K <= x || x + (int64_t)E * max_m * K <= out,
              MOE_EINVAL, "moe_fp8_requant: out partially overlaps x (only out == x is allowed)");
  moe_requant_config c;
  if (cfg) {
    c = *cfg;
    MOE_REQUIRE(c.workgroups >= 1 && (c.unroll == 1 || c.unroll == 2 || c.unroll == 4), MOE_EINVAL,
                "moe_fp8_requant: config workgroups=%d unroll=%d (need >= 1 and 1, 2 or 4)",
                c.workgroups, c.unroll);
  } else {
    const int rc = moe_fp8_requant_choose(E, max_m, K, 0, device_cu_count(), &c);
    if (rc) return rc;
  }
  const int ch = (int)chunks;
  if (E <= 64)
    launch_pmax<1>(c.unroll, c.workgroups, stream, x, out, scales, scale_stride_e, scale_stride_m,
                   scale_stride_g, masked_m, tensor_scale, E, max_m, K, group_size, ch);
  else if (E <= 256)
    launch_pmax<4>(c.unroll, c.workgroups, stream, x, out, scales, scale_stride_e, scale_stride_m,
                   scale_stride_g, masked_m, tensor_scale, E, max_m, K, group_size, ch);
  else
    launch_pmax<16>(c.unroll, c.workgroups, stream, x, out, scales, scale_stride_e, scale_stride_m,
                    scale_stride_g, masked_m, tensor_scale, E, max_m, K, group_size, ch);
  return check_launch("moe_fp8_requant");
}
