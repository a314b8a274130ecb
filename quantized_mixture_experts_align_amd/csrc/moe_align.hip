// Route-and-align: stable counting sort of the top-k assignments by local expert.
//
// The Muse Spark experiment maps global ids to local ones with expert_map (-1 off the local
// range) and calls moe_align_block_size(local_ids, block_size_m, ...), which returns the slot
// ids grouped by expert and padded per expert to a multiple of the block size, one expert id
// per block, and the padded total.  Here the routing is fused in (a range test), off-slice
// assignments are dropped, and the order inside an expert is ascending slot id, so the result
// is unique and reproducible.
//
// One or more workgroups of 16 waves; workgroup g owns the slots [g*span, (g+1)*span) and
// wave w of it a contiguous chunk of those, a multiple of 64 long.
//   0. totals:  with several workgroups, each one counts the whole batch per expert -- the slots
//               before its span, then the rest, each wave into its own LDS row, rows summed --
//               (one read of every id from L2 per workgroup: no workspace and no communication
//               between workgroups, and every workgroup derives the same segment starts)
//   1. count:   LDS histogram cnt[w][e] of the span (atomics only add; the totals do not depend
//               on order)
//   2. scan:    per expert, exclusive scan over the waves (a 16-lane segmented shuffle scan per
//               expert) -> offset of wave w inside the span's part of the expert's segment;
//               padded totals scanned over experts -> segment starts (up to 64 experts: wave 0
//               alone does both, one lane per expert, behind a single barrier)
//   3. scatter: each wave walks its chunk in order, 64 slots at a time; the rank of a lane among
//               the lanes of its batch with the same expert comes from ballots over the bits of
//               the expert id (a wave multi-split), so the write position is
//               seg[e] + before[e] + off[w][e] + rank, strictly in slot order.  A chunk of up to
//               64 * kAlignUnroll slots keeps its ids in registers from step 1 (one read of ids)
//   4. fill:    padding entries (in parallel over expert x position) and the tail get the
//               sentinel, block -> expert by binary search over the segment starts; these index
//               ranges are split over the workgroups
//   5. schedule (moe_align_sched only): the position of every live block in the GEMM's block
//               order, computed in each workgroup from the per-expert totals alone (so all agree):
//               an expert's last block with fewer than C = ceil(B/16) live 16-slot groups (a
//               "short" block) sets bit (C-1-groups) * n_local + e of a key bitmap, and a short
//               block's position is the number of full-class blocks plus the set bits below its key;
//               any other block keeps its index minus the short blocks of the experts before it
#include "moe_internal.h"

namespace moe {

constexpr int kAlignWaves = 16;
constexpr int kAlignThreads = kAlignWaves * 64;
constexpr int kAlignMaxLocal = 512;
constexpr int kAlignUnroll = 8;
// Batches of more slots than this are split over workgroups of kAlignSpan slots each.  Measured
// (kernel trace, NVFP4 EP8 slice): 32768 slots 30.6 -> 9.6 us, 8192 slots 9.0 -> 6.7 us (32
// experts) and 14.4 -> 9.3 us (128 experts), 186368 slots 25.5 us.
constexpr int kAlignSingleMax = 4096;
constexpr int kAlignSpan = 2048;
// At most this many workgroups (longer spans beyond 512K slots): each counts the whole batch, so
// the ids are read workgroups x numel times in all.
constexpr int kAlignMaxGroups = 256;
// key bitmap of the block schedule: (16-slot classes below full) x experts, at most 15 x 512 bits
constexpr int kSchedKeyWords = (15 * kAlignMaxLocal + 31) / 32;

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int32_t numel, int32_t start, int32_t n_local, int32_t B,
    int32_t cap, int32_t cap_blocks, int32_t span, int32_t* __restrict__ sorted,
    int32_t* __restrict__ eids, int32_t* __restrict__ ntpp, int32_t* __restrict__ slot_local,
    int32_t* __restrict__ border) {
  __shared__ int32_t cnt[kAlignWaves * kAlignMaxLocal];  // per wave and expert
  __shared__ int32_t seg[kAlignMaxLocal + 1];            // segment start of each expert
  __shared__ int32_t tot[kAlignMaxLocal];                // live slots of each expert (whole batch)
  __shared__ int32_t bef[kAlignMaxLocal];                // live slots of each expert before the span
  __shared__ int32_t wave_sum[kAlignWaves];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int G = (int)gridDim.x, g = (int)blockIdx.x;
  const int s0 = (int)min((int64_t)numel, (int64_t)g * span), s1 = (int)min((int64_t)numel, (int64_t)s0 + span);
  auto local_of = [&](int id) { return (id >= start && id - start < n_local) ? id - start : -1; };

  int nbits = 0;
  while ((1 << nbits) < n_local) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // lanes of a 64-slot batch with the same local expert as this lane (live lanes only): ballots
  // over the bits of the expert id (a wave multi-split)
  auto same_expert = [&](int le) {
    const bool live = le >= 0;
    uint64_t same = __ballot(live);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = live && ((le >> b) & 1);
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    return same;
  };

  int32_t* my_cnt = cnt + w * n_local;
  // per-wave counts of the slots [i0, i1) into the wave's own row (per-lane LDS atomics: lanes of
  // one wave only ever meet on a counter), four 64-slot batches' ids in flight
  auto count_rows = [&](int i0, int i1) {
    for (int i = lane; i < n_local; i += 64) my_cnt[i] = 0;
    __builtin_amdgcn_wave_barrier();
    constexpr int kU = 4;
    for (int base = i0 + w * 64; base < i1; base += kU * kAlignThreads) {
      int idq[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + u * kAlignThreads + lane;
        idq[u] = i < i1 ? ids[i] : -1;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int le = local_of(idq[u]);
        if (le >= 0) atomicAdd(&my_cnt[le], 1);
      }
    }
    __syncthreads();
  };
  if (G > 1) {
    // the slots before the span, then the rest of the batch; the rows summed per expert
    count_rows(0, s0);
    for (int e = tid; e < n_local; e += kAlignThreads) {
      int t = 0;
      for (int v = 0; v < kAlignWaves; ++v) t += cnt[v * n_local + e];
      bef[e] = t;
    }
    __syncthreads();
    count_rows(s0, numel);
    for (int e = tid; e < n_local; e += kAlignThreads) {
      int t = bef[e];
      for (int v = 0; v < kAlignWaves; ++v) t += cnt[v * n_local + e];
      tot[e] = t;
    }
    __syncthreads();
  } else {
    for (int e = tid; e < n_local; e += kAlignThreads) bef[e] = 0;
  }
  // each wave zeroes and then counts into its own row only: a wave barrier suffices there
  for (int i = lane; i < n_local; i += 64) my_cnt[i] = 0;
  __builtin_amdgcn_wave_barrier();

  // every wave owns a chunk of the span (the scatter is serial per 64-slot batch within a wave,
  // so short chunks are faster even when most waves are idle)
  const int nwv = kAlignWaves;
  const int len = s1 - s0;
  const int per = ((len + nwv - 1) / nwv + 63) & ~63;
  const int c0 = min(s1, s0 + w * per), c1 = min(s1, c0 + per);
  const bool keep = per <= 64 * kAlignUnroll;  // the chunk's ids stay in registers

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
        if (G > 1) t = tot[lane];
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
        if (v == 15 && G == 1) tot[e] = x;
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
      const uint64_t same = same_expert(le);
      if (le >= 0) {
        const int rank = __popcll(same & lt_mask);
        const int before = my_cnt[le];
        sorted[seg[le] + bef[le] + before + rank] = i;
        if ((same >> lane) == 1ull) my_cnt[le] = before + __popcll(same);  // last lane of the group
      }
      __builtin_amdgcn_wave_barrier();
    }
  }

  // padding of each expert's last block (expert x position in parallel), then the tail; each
  // index range split over the workgroups
  const int gt = g * kAlignThreads + tid, gstride = G * kAlignThreads;
  for (int i = gt; i < n_local * B; i += gstride) {
    const int e = i / B, p = seg[e] + tot[e] + (i - e * B);
    if (p < seg[e + 1]) sorted[p] = numel;
  }
  const int total = seg[n_local];
  for (int p = total + gt; p < cap; p += gstride) sorted[p] = numel;

  // block schedule: key bitmap of the short blocks, their experts, and prefix counts of the keys
  __shared__ uint32_t key_bits[kSchedKeyWords];
  __shared__ uint32_t short_bits[kAlignMaxLocal / 32];
  __shared__ int32_t key_pre[kSchedKeyWords + 1];
  const int C = (B + 15) >> 4;                 // 16-slot groups of a full block
  const int nkw = ((C - 1) * n_local + 31) >> 5;
  // the short last block of expert e: its key, or -1
  auto short_key = [&](int e) {
    const int r = tot[e] % B, lg = (r + 15) >> 4;
    return (r > 0 && lg < C) ? (C - 1 - lg) * n_local + e : -1;
  };
  if (border) {
    for (int i = tid; i < nkw; i += kAlignThreads) key_bits[i] = 0u;
    for (int i = tid; i < kAlignMaxLocal / 32; i += kAlignThreads) short_bits[i] = 0u;
    __syncthreads();
    for (int e = tid; e < n_local; e += kAlignThreads) {
      const int k = short_key(e);
      if (k >= 0) {
        atomicOr(&key_bits[k >> 5], 1u << (k & 31));
        atomicOr(&short_bits[e >> 5], 1u << (e & 31));
      }
    }
    __syncthreads();
    if (w == 0) {
      int run = 0;
      for (int base = 0; base < nkw; base += 64) {
        const int i = base + lane;
        const int c = i < nkw ? __popc(key_bits[i]) : 0;
        int x = c;
        for (int d = 1; d < 64; d <<= 1) {
          const int o = __shfl_up(x, d);
          if (lane >= d) x += o;
        }
        if (i < nkw) key_pre[i] = run + x - c;
        run += __shfl(x, 63);
      }
      if (lane == 0) key_pre[nkw] = run;
    }
    __syncthreads();
  }
  const int nb_live = total / B;
  const int n_top = border ? nb_live - key_pre[nkw] : 0;  // blocks of the full class
  for (int b = gt; b < cap_blocks; b += gstride) {
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
    if (border) {
      if (b >= nb_live) {
        border[b] = -1;  // (positions from nb_live on hold no block)
      } else {
        const int k = (b + 1) * B == seg[e + 1] ? short_key(e) : -1;
        int pos;
        if (k >= 0) {
          pos = n_top + key_pre[k >> 5] + __popc(key_bits[k >> 5] & ((1u << (k & 31)) - 1u));
        } else {
          int before = __popc(short_bits[e >> 5] & ((1u << (e & 31)) - 1u));
          for (int j = 0; j < (e >> 5); ++j) before += __popc(short_bits[j]);
          pos = b - before;
        }
        border[pos] = b;
      }
    }
  }
  if (gt == 0) *ntpp = total;
}

}  // namespace moe

using namespace moe;

static int align_launch(const int32_t* topk_ids, int64_t M, int32_t top_k, int32_t expert_start,
                        int32_t n_local, int32_t block_m, int32_t* sorted_token_ids, int32_t* expert_ids,
                        int32_t* num_tokens_post_padded, int32_t* slot_local_ids, bool sched,
                        int32_t* block_order, hipStream_t stream) {
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
  MOE_REQUIRE(!sched || block_order || cap_blocks == 0, MOE_EINVAL, "moe_align_sched: null block_order");
  const int64_t numel = M * top_k;
  const int32_t span = numel <= kAlignSingleMax
                           ? (int32_t)std::max<int64_t>(numel, 1)
                           : (int32_t)std::max<int64_t>(kAlignSpan, (numel + kAlignMaxGroups - 1) / kAlignMaxGroups);
  const unsigned grid = (unsigned)std::max<int64_t>(1, (numel + span - 1) / span);
  hipLaunchKernelGGL(align_kernel, dim3(grid), dim3(kAlignThreads), 0, stream, topk_ids, (int32_t)numel,
                     expert_start, n_local, block_m, (int32_t)cap, (int32_t)cap_blocks, span, sorted_token_ids,
                     expert_ids, num_tokens_post_padded, slot_local_ids, block_order);
  return check_launch("moe_align");
}

extern "C" int moe_align(const int32_t* topk_ids, int64_t M, int32_t top_k, int32_t expert_start,
                         int32_t n_local, int32_t block_m, int32_t* sorted_token_ids,
                         int32_t* expert_ids, int32_t* num_tokens_post_padded,
                         int32_t* slot_local_ids, hipStream_t stream) {
  return align_launch(topk_ids, M, top_k, expert_start, n_local, block_m, sorted_token_ids, expert_ids,
                      num_tokens_post_padded, slot_local_ids, false, nullptr, stream);
}

extern "C" int moe_align_sched(const int32_t* topk_ids, int64_t M, int32_t top_k, int32_t expert_start,
                               int32_t n_local, int32_t block_m, int32_t* sorted_token_ids,
                               int32_t* expert_ids, int32_t* num_tokens_post_padded,
                               int32_t* slot_local_ids, int32_t* block_order, hipStream_t stream) {
  return align_launch(topk_ids, M, top_k, expert_start, n_local, block_m, sorted_token_ids, expert_ids,
                      num_tokens_post_padded, slot_local_ids, true, block_order, stream);
}
