// Route-and-align: stable counting sort of the top-k assignments by local expert.
//
// The Muse Spark experiment maps global ids to local ones with expert_map (-1 off the local
// range) and calls moe_align_block_size(local_ids, block_size_m, ...), which returns the slot
// ids grouped by expert and padded per expert to a multiple of the block size, one expert id
// per block, and the padded total.  Here the routing is fused in (a range test), off-slice
// assignments are dropped, and the order inside an expert is ascending slot id, so the result
// is unique and reproducible.
//
// One workgroup of 16 waves; wave w owns a contiguous chunk of slots, a multiple of 64 long.
//   1. count:   LDS histogram cnt[w][e] (atomics only add; the totals do not depend on order)
//   2. scan:    per expert, exclusive scan over the waves (a 16-lane segmented shuffle scan per
//               expert) -> offset of wave w inside the expert's segment and the expert's total;
//               padded totals scanned over experts -> segment starts (up to 64 experts: wave 0
//               alone does both, one lane per expert, behind a single barrier)
//   3. scatter: each wave walks its chunk in order, 64 slots at a time; the rank of a lane among
//               the lanes of its batch with the same expert comes from ballots over the bits of
//               the expert id (a wave multi-split), so the write position is
//               seg[e] + off[w][e] + rank, strictly in slot order.  A chunk of up to
//               64 * kAlignUnroll slots keeps its ids in registers from step 1 (one read of ids)
//   4. fill:    padding entries (in parallel over expert x position) and the tail get the
//               sentinel, block -> expert by binary search over the segment starts
#include "moe_internal.h"

namespace moe {

constexpr int kAlignWaves = 16;
constexpr int kAlignThreads = kAlignWaves * 64;
constexpr int kAlignMaxLocal = 512;
constexpr int kAlignUnroll = 8;

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int32_t numel, int32_t start, int32_t n_local, int32_t B,
    int32_t cap, int32_t cap_blocks, int32_t* __restrict__ sorted, int32_t* __restrict__ eids,
    int32_t* __restrict__ ntpp, int32_t* __restrict__ slot_local) {
  __shared__ int32_t cnt[kAlignWaves * kAlignMaxLocal];  // per wave and expert
  __shared__ int32_t seg[kAlignMaxLocal + 1];            // segment start of each expert
  __shared__ int32_t tot[kAlignMaxLocal];                // live slots of each expert
  __shared__ int32_t wave_sum[kAlignWaves];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  // every wave owns a chunk (the scatter is serial per 64-slot batch within a wave, so short
  // chunks are faster even when most waves are idle)
  const int nwv = kAlignWaves;
  // each wave zeroes and then counts into its own row only: a wave barrier suffices here
  for (int i = lane; i < n_local; i += 64) cnt[w * n_local + i] = 0;
  __builtin_amdgcn_wave_barrier();

  // chunk of wave w: [c0, c1), a multiple of 64 slots long (empty for waves >= nwv)
  const int per = ((numel + nwv - 1) / nwv + 63) & ~63;
  const int c0 = w < nwv ? min(numel, w * per) : numel, c1 = w < nwv ? min(numel, c0 + per) : numel;
  const bool keep = per <= 64 * kAlignUnroll;  // the chunk's ids stay in registers
  int32_t* my_cnt = cnt + w * n_local;

  auto local_of = [&](int id) { return (id >= start && id - start < n_local) ? id - start : -1; };
  // (ids are read kAlignUnroll batches at a time so their load latencies overlap)
  int idv[kAlignUnroll];
  for (int base = c0; base < c1; base += 64 * kAlignUnroll) {
#pragma unroll
    for (int u = 0; u < kAlignUnroll; ++u) {
      const int i = base + 64 * u + lane;
      idv[u] = i < c1 ? ids[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignUnroll; ++u) {
      const int i = base + 64 * u + lane;
      if (i >= c1) break;
      const int le = local_of(idv[u]);
      if (slot_local) slot_local[i] = le;
      if (le >= 0) atomicAdd(&my_cnt[le], 1);
    }
  }
  __syncthreads();

  if (n_local <= 64) {
    // few experts: wave 0 alone, lane e = expert e -- its waves' counts in wave order (exclusive
    // prefix) and total, then the padded totals scanned over the lanes; one barrier instead of three
    if (w == 0) {
      int t = 0;
      if (lane < n_local) {
        // all counts first, then the prefixes: interleaved, every read would wait for the
        // previous write (the compiler cannot tell the rows apart)
        int c[kAlignWaves];
#pragma unroll
        for (int v = 0; v < kAlignWaves; ++v) c[v] = cnt[v * n_local + lane];
#pragma unroll
        for (int v = 0; v < kAlignWaves; ++v) {
          cnt[v * n_local + lane] = t;
          t += c[v];
        }
      }
      const int p = lane < n_local ? (t + B - 1) / B * B : 0;
      int incl = p;
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
      }
      if (lane < n_local) {
        tot[lane] = t;
        seg[lane] = incl - p;
      }
      if (lane == n_local - 1) seg[n_local] = incl;
    }
    __syncthreads();
  } else {
    // per expert: exclusive scan of the waves' counts (wave order) and the total; lanes
    // 16 j .. 16 j + 15 of a wave hold waves 0..15 of one expert
    for (int base = 0; base < n_local * 16; base += kAlignThreads) {
      const int i = base + tid, e = i >> 4, v = i & 15;
      const int c = (e < n_local && v < nwv) ? cnt[v * n_local + e] : 0;
      int x = c;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const int o = __shfl_up(x, d, 16);
        if (v >= d) x += o;
      }
      if (e < n_local) {
        if (v < nwv) cnt[v * n_local + e] = x - c;
        if (v == 15) tot[e] = x;
      }
    }
    __syncthreads();

    // exclusive scan of the padded totals over experts (n_local <= 512 < threads)
    {
      const int p = tid < n_local ? (tot[tid] + B - 1) / B * B : 0;
      int incl = p;
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
      }
      if (lane == 63) wave_sum[w] = incl;
      __syncthreads();
      int before = 0;
      for (int v = 0; v < w; ++v) before += wave_sum[v];
      incl += before;
      if (tid < n_local) seg[tid] = incl - p;
      if (tid == n_local - 1) seg[n_local] = incl;
    }
    __syncthreads();
  }

  // scatter in slot order
  int nbits = 0;
  while ((1 << nbits) < n_local) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = c0; base < c1; base += 64 * kAlignUnroll) {
    if (!keep) {
#pragma unroll
      for (int u = 0; u < kAlignUnroll; ++u) {
        const int i = base + 64 * u + lane;
        idv[u] = i < c1 ? ids[i] : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < kAlignUnroll; ++u) {
      const int i = base + 64 * u + lane;
      if (base + 64 * u >= c1) break;  // uniform: the wave's chunk has ended
      const int le = i < c1 ? local_of(idv[u]) : -1;
      const bool live = le >= 0;
      uint64_t same = __ballot(live);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = live && ((le >> b) & 1);
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
      }
      if (live) {
        const int rank = __popcll(same & lt_mask);
        const int before = my_cnt[le];
        sorted[seg[le] + before + rank] = i;
        if ((same >> lane) == 1ull) my_cnt[le] = before + __popcll(same);  // last lane of the group
      }
      __builtin_amdgcn_wave_barrier();
    }
  }

  // padding of each expert's last block (expert x position in parallel), then the tail
  for (int i = tid; i < n_local * B; i += kAlignThreads) {
    const int e = i / B, p = seg[e] + tot[e] + (i - e * B);
    if (p < seg[e + 1]) sorted[p] = numel;
  }
  const int total = seg[n_local];
  for (int p = total + tid; p < cap; p += kAlignThreads) sorted[p] = numel;
  for (int b = tid; b < cap_blocks; b += kAlignThreads) {
    int e = -1;
    if (b * B < total) {
      int lo = 0, hi = n_local;  // first index with seg[idx] > b*B, minus one
      const int x = b * B;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (seg[mid + 1] <= x) lo = mid + 1; else hi = mid;
      }
      e = lo;
    }
    eids[b] = e;
  }
  if (tid == 0) *ntpp = total;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_align(const int32_t* topk_ids, int64_t M, int32_t top_k, int32_t expert_start,
                         int32_t n_local, int32_t block_m, int32_t* sorted_token_ids,
                         int32_t* expert_ids, int32_t* num_tokens_post_padded,
                         int32_t* slot_local_ids, hipStream_t stream) {
  MOE_REQUIRE(M >= 0 && top_k >= 1 && top_k <= 64, MOE_EINVAL, "moe_align: M=%lld top_k=%d",
              (long long)M, top_k);
  MOE_REQUIRE(n_local >= 1 && n_local <= kAlignMaxLocal, MOE_EUNSUPPORTED,
              "moe_align: n_local=%d outside 1..%d", n_local, kAlignMaxLocal);
  MOE_REQUIRE(block_m >= 1 && block_m <= 256, MOE_EUNSUPPORTED, "moe_align: block_m=%d outside 1..256",
              block_m);
  MOE_REQUIRE(expert_start >= 0, MOE_EINVAL, "moe_align: expert_start=%d", expert_start);
  int64_t cap = 0, cap_blocks = 0;
  int rc = moe_align_capacity(M, top_k, n_local, block_m, &cap, &cap_blocks);
  if (rc) return rc;
  MOE_REQUIRE(cap < (int64_t)1 << 30, MOE_EUNSUPPORTED, "moe_align: %lld entries is too many",
              (long long)cap);
  MOE_REQUIRE(num_tokens_post_padded && ((sorted_token_ids && expert_ids) || cap == 0), MOE_EINVAL,
              "moe_align: null output pointer");
  MOE_REQUIRE(topk_ids || M == 0, MOE_EINVAL, "moe_align: null topk_ids");
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, stream, topk_ids, (int32_t)(M * top_k),
                     expert_start, n_local, block_m, (int32_t)cap, (int32_t)cap_blocks, sorted_token_ids,
                     expert_ids, num_tokens_post_padded, slot_local_ids);
  return check_launch("moe_align");
}
