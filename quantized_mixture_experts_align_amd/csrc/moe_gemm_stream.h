// gemm_stream: grouped W4A16 GEMM for align blocks of at most 16 slots (decode batches), whose
// cost is streaming the touched experts' weights from HBM.  Built to keep an uninterrupted
// stream of weight loads in flight.
//
// Work item = (live align block, strip of NG 16-row weight tiles).  A persistent workgroup walks
// a contiguous range of items; its KS waves split K (wave w owns k-tiles [KT w/KS, KT (w+1)/KS)).
// Each wave runs ONE flat sequence of k-steps over all of its items with a register ring D steps
// deep (per step: the NG tiles' codes -- 8 B per lane, one 512-B wave load per tile --, their
// group scales and the step's 16-slot activation column), so the next item's first loads are in
// flight while the previous item finishes: there is no per-item pipeline drain.  Everything an
// item needs besides the streamed operands (expert, slot rows, NVFP4 global scale, bias) is
// staged in LDS when the workgroup starts (the launch gives no workgroup more than kWin items),
// so inside the stream nothing waits on a vector-memory load other than the ring's own (a load
// of bias in the epilogue would wait for every weight load issued before it).
//
// Per step and tile each lane feeds one v_mfma_f32_16x16x32_bf16 per k-substep: weights as the A
// operand (rows = output features), the 16 slots of the block as the B operand (columns; dead
// columns read token 0 and are never stored).  At an item's last step the waves' partial sums are
// added through LDS in a fixed wave order (double-buffered by item parity: one barrier per item)
// and wave 0 applies global scale, bias and (fused gate/up) the activation, and writes the
// block's live rows.
#pragma once

#include "moe_gemm_common.h"

namespace moe {

constexpr int kWin = 32;  // most items per workgroup (their metadata is staged in LDS)

// LDS-only barrier: waits for this wave's LDS traffic, not for its vector-memory loads (the ring).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wave 0's part: the align of the slots in NB 64-slot batches (numel <= 64 * NB), one slot per
// lane in each batch.
template <int NB>
__device__ void fused_align_wave(const GemmArgs& a, int* f_rows, int* f_be, int* f_nblk) {
  const int lane = (int)threadIdx.x & 63, B = a.block_m, numel = a.numel;
  int le[NB];
  bool live[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int s = 64 * j + lane;
    const int id = s < numel ? a.topk_ids[s] : -1;
    live[j] = s < numel && id >= a.expert_start && id - a.expert_start < a.E;
    le[j] = live[j] ? id - a.expert_start : -1;
  }
  // the slots of batch jj routed to local expert e (e is this lane's own; the ballots over the
  // bits of the batch's expert ids are the same for every lane)
  auto same_in = [&](int jj, int e) {
    uint64_t m = __ballot(live[jj]);
    for (int b = 0; (1 << b) < a.E; ++b) {
      const uint64_t mb = __ballot(live[jj] && ((le[jj] >> b) & 1));
      m &= ((e >> b) & 1) ? mb : ~mb;
    }
    return m;
  };
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int r[NB], nbe[NB];
  bool first[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    int before = 0, count = 0;   // the expert's slots in earlier batches / in all batches
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) {
      const uint64_t m = same_in(jj, le[j]);
      if (jj < j) before += __popcll(m);
      if (jj == j) before += __popcll(m & below);
      count += __popcll(m);
    }
    r[j] = before;                          // rank among the expert's slots
    nbe[j] = (count + B - 1) / B;           // blocks of the expert
    first[j] = live[j] && r[j] == 0;
  }
  // blocks of the experts before each slot's: a walk over the first slot of every live expert
  int bs[NB], tot = 0;
#pragma unroll
  for (int j = 0; j < NB; ++j) bs[j] = 0;
#pragma unroll
  for (int jj = 0; jj < NB; ++jj) {
    uint64_t fm = __ballot(first[jj]);
    while (fm) {
      const int q = __builtin_ctzll(fm);
      fm &= fm - 1;
      const int lej = __shfl(le[jj], q), nj = __shfl(nbe[jj], q);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (lej < le[j]) bs[j] += nj;
      tot += nj;
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (live[j]) f_rows[(bs[j] + r[j] / B) * 16 + r[j] % B] = 64 * j + lane;
    if (first[j])
      for (int t = 0; t < nbe[j]; ++t) f_be[bs[j] + t] = le[j];
    if (blockIdx.x == 0 && 64 * j + lane < numel) a.slot_local_out[64 * j + lane] = le[j];
  }
  if (lane == 0) *f_nblk = tot;
}

// Route-and-align of at most kFusedAlignSlots slots, computed by wave 0, one slot per lane in each
// 64-slot batch (the same result as moe_align: local expert = id - start inside [start, start + E),
// else the slot is dropped; slots grouped by ascending expert, ascending slot order inside an
// expert, each expert's run padded to whole blocks of B rows with the sentinel numel).
//   f_rows[b * 16 + r] = slot of row r of block b (numel for padding), f_be[b] = its expert,
//   returns the block count.  Workgroup 0 also writes sorted_out[cap], eids_out[cap_blocks]
//   (-1 past the last block), *ntpp_out and slot_local_out[numel].  Every thread calls it.
template <int NB>
__device__ int fused_align(const GemmArgs& a, int* f_rows, int* f_be, int* f_nblk) {
  const int tid = (int)threadIdx.x, B = a.block_m, numel = a.numel;
  // (a block holds at least one live slot, so at most numel blocks are ever read)
  for (int p = tid; p < min(numel, 64 * NB) * 16; p += (int)blockDim.x) f_rows[p] = numel;
  __syncthreads();
  if (tid < 64) fused_align_wave<NB>(a, f_rows, f_be, f_nblk);
  __syncthreads();
  const int nb = *f_nblk;
  if (blockIdx.x == 0) {
    const int total = nb * B;
    for (int p = tid; p < a.cap; p += (int)blockDim.x) a.sorted_out[p] = p < total ? f_rows[(p / B) * 16 + p % B] : numel;
    for (int b = tid; b < a.cap_blocks; b += (int)blockDim.x) a.eids_out[b] = b < nb ? f_be[b] : -1;
    if (tid == 0) *a.ntpp_out = total;
  }
  return nb;
}

template <int QT, bool BIAS, int NG, int KS, int ACT, int FA, bool CMB>
__global__ __launch_bounds__(64 * KS) void gemm_stream_kernel(GemmArgs a) {
  static_assert(!act_paired<ACT>() || NG % 2 == 0, "the fused gated epilogue pairs gate and up tiles");
  static_assert(!CMB || (ACT == kActNone && !FA), "the fused weighted sum follows a plain projection");
  constexpr int NGA = act_paired<ACT>() ? NG / 2 : NG;
  constexpr int D = NG >= 4 ? 4 : 8;  // ring depth (k-steps): about 9 KB of weights per wave
  __shared__ int t_e[kWin];
  __shared__ float t_gs[kWin];
  __shared__ int t_row[kWin][16];                  // slot of each column of the block, -1 = dead
  __shared__ uint16_t t_bias[BIAS ? kWin : 1][NG][16];
  __shared__ f32x4_t red[2][KS > 1 ? KS - 1 : 1][NG][64];

  // the wave index is uniform: keep it (and everything derived from it) in scalar registers
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int NT = a.N / kTileN, KT = a.K / kTileK;
  const int NTA = act_paired<ACT>() ? NT / 2 : NT;  // tiles to assign (gate tiles if fused)
  const int NS = (NTA + NGA - 1) / NGA;           // strips per block
  const int B = a.block_m;
  // fused align (FA = its 64-slot batches, 0 = none)
  __shared__ int f_rows[FA ? FA * 64 * 16 : 1];
  __shared__ int f_be[FA ? FA * 64 : 1];
  __shared__ int f_nblk;
  const int nblocks = [&] {
    if constexpr (FA > 0) return fused_align<FA>(a, f_rows, f_be, &f_nblk);
    else return *a.ntpp / B;
  }();
  const int items = nblocks * NS;
  if constexpr (CMB) {  // a token without a live slot sums to zero: no item ever reaches it
    for (int t = blockIdx.x; t < a.cmb_ntok; t += gridDim.x) {
      bool any = false;
      for (int j = 0; j < a.cmb_k; ++j) any |= a.cmb_live[(int64_t)t * a.cmb_k + j] >= 0;
      if (!any)
        for (int c = tid; c < a.N; c += 64 * KS) a.cmb_out[(int64_t)t * a.cmb_ldo + c] = 0;
    }
  }
  // items split evenly over the whole grid (every workgroup gets floor or ceil of the mean, at
  // most kWin by the launch), so that no workgroup idles while others take an extra item
  const int i0 = (int)((int64_t)blockIdx.x * items / (int)gridDim.x);
  const int i1 = (int)((int64_t)(blockIdx.x + 1) * items / (int)gridDim.x);
  if (i0 >= i1) return;
  const int kt0 = KT * w / KS, kt1 = KT * (w + 1) / KS, L = kt1 - kt0;  // L >= 1: KT >= KS
  const int m = lane & 15, j8 = 8 * (lane >> 4);

  auto tile_of = [&](int strip, int g) {
    const int t = min(strip * NGA + (g < NGA ? g : g - NGA), NTA - 1);
    return g < NGA ? t : t + NTA;
  };

  int par = 0;
  {
    const int wb = i0, wn = min(kWin, i1 - i0);  // (the min only guards the LDS table)
    for (int t = tid; t < wn * 16; t += 64 * KS) {
      const int q = t >> 4, mm = t & 15, b = (wb + q) / NS;
      int s = -1;
      if (mm < B) {
        s = FA ? f_rows[b * 16 + mm] : a.sorted[(int64_t)b * B + mm];
        if (s < 0 || s >= a.numel) s = -1;
      }
      t_row[q][mm] = s;
      if (mm == 0) {
        const int e = FA ? f_be[b] : a.eids[b];
        const bool ok = e >= 0 && e < a.E;
        t_e[q] = ok ? e : -1;
        t_gs[q] = (QT == MOE_Q_NVFP4_G16 && ok) ? a.gs[e] : 1.0f;
      }
    }
    if constexpr (BIAS) {
      for (int t = tid; t < wn * NG * 16; t += 64 * KS) {
        const int q = t / (NG * 16), g = (t >> 4) % NG, r = t & 15;
        const int it = wb + q, b = it / NS, e = FA ? f_be[b] : a.eids[b];
        t_bias[q][g][r] = (e >= 0 && e < a.E) ? a.bias[(int64_t)e * a.N + tile_of(it - b * NS, g) * kTileN + r] : 0;
      }
    }
    __syncthreads();

    // ---- issue side: the step (iq, ikt) whose operands are loaded next
    int iq = 0, ikt = kt0;
    const u32x2_t* wp[NG];
    const uint8_t* sp[NG];
    const uint16_t* xp;
    auto enter = [&](int q) {
      const int it = wb + q, b = it / NS, strip = it - b * NS;
      const int e = max(t_e[q], 0);  // a dead item still loads valid memory; nothing is stored
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int64_t tile = (int64_t)e * NT + tile_of(strip, g);
        wp[g] = reinterpret_cast<const u32x2_t*>(a.codes + tile * KT * kTileBytes) + lane;
        sp[g] = a.scales + tile * (pair_grouped(QT) ? KT / 2 : KT) * scale_step_bytes(QT);
      }
      const int s = t_row[q][m];
      xp = a.A + (int64_t)(s >= 0 ? s / a.top_k : 0) * a.lda + j8;
    };
    u32x2_t rq[D][NG];
    TileScale<QT> rs[D][NG];
    u32x4_t rx[D][2];
    // load the issue step into ring slot u, then advance; past the wave's last step the last step
    // is loaded again (valid addresses, unused), which keeps every slot's load count the same
    auto issue = [&](int u) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        rq[u][g] = wp[g][(int64_t)ikt * 64];
        rs[u][g].load(sp[g], ikt, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) rx[u][i] = *reinterpret_cast<const u32x4_t*>(xp + ikt * kTileK + 32 * i);
      if (++ikt == kt1) {
        if (iq + 1 < wn) {
          ++iq;
          ikt = kt0;
          enter(iq);
        } else {
          ikt = kt1 - 1;
        }
      }
    };

    // ---- compute side
    f32x4_t acc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int cq = 0, cs = 0;
    // Fused weighted sum (wave 0, once the workgroup's items are all stored): publish the rows
    // (one release fence: a fence waits for every load in flight, so it is kept out of the
    // streaming loop), count each item's arrival at its tokens' (token, strip) counters, and let
    // the arrival that completes a token's live slots sum them, in slot order, exactly as the
    // combine kernel does.  Release fence -> counter RMW -> acquire fence: every earlier arrival's
    // rows are visible to the completing wave, whichever XCD wrote them.  The completing lane
    // resets its counter.
    auto combine_all = [&](int nq) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const int g = lane >> 4, r = lane & 15;  // lane -> column (tile g of the strip, row r)
      for (int q = 0; q < nq; ++q) {
        const int strip = (wb + q) % NS, e = t_e[q], s = t_row[q][m];
        bool done = false;
        int tok = 0;
        if (lane < 16 && e >= 0 && s >= 0) {
          tok = s / a.cmb_k;
          int live = 0;
          for (int j = 0; j < a.cmb_k; ++j) live += a.cmb_live[(int64_t)tok * a.cmb_k + j] >= 0;
          int* c = a.cmb_cnt + (int64_t)tok * NS + strip;
          if (__hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == live - 1) {
            done = true;
            __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        uint64_t dm = __ballot(done);
        if (dm == 0) continue;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        const bool col_ok = g < NG && strip * NG + g < NT;
        const int col = (strip * NG + g) * kTileN + r;
        while (dm) {
          const int src = __ffsll((unsigned long long)dm) - 1;
          dm &= dm - 1;
          const int t = __shfl(tok, src);
          if (!col_ok) continue;
          float acc = 0.f;
          for (int j = 0; j < a.cmb_k; ++j) {
            const int64_t slot = (int64_t)t * a.cmb_k + j;
            if (a.cmb_live[slot] < 0) continue;
            acc = fmaf(a.cmb_gw[slot], bf16_to_f32(a.C[slot * a.ldc + col]), acc);
          }
          acc *= a.cmb_rsf;
          a.cmb_out[(int64_t)t * a.cmb_ldo + col] = f32_to_bf16(acc);
        }
      }
    };
    auto finish = [&](int q) {  // the item's partial sums are complete in every wave
      if constexpr (KS > 1) {
        if (w > 0)
#pragma unroll
          for (int g = 0; g < NG; ++g) red[par][w - 1][g][lane] = acc[g];
        lds_barrier();
        if (w == 0)
          for (int v = 0; v < KS - 1; ++v)
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[g] += red[par][v][g][lane];
        par ^= 1;
      }
      const int e = t_e[q], s = t_row[q][m];
      if (w == 0 && e >= 0 && s >= 0) {
        const int strip = (wb + q) % NS;
        const float gs = t_gs[q];
        const int r0 = 4 * (lane >> 4);  // D[n][m]: this lane holds rows r0 .. r0+3 of column m
        auto fin = [&](float v, int g, int r) {
          if constexpr (QT == MOE_Q_NVFP4_G16) v *= gs;
          if constexpr (BIAS) v += bf16_to_f32(t_bias[q][g][r]);
          return v;
        };
#pragma unroll
        for (int g = 0; g < NGA; ++g) {
          if (strip * NGA + g >= NTA) break;
          float v[4];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            v[qq] = fin(acc[g][qq], g, r0 + qq);
            if constexpr (act_paired<ACT>()) v[qq] = fused_act<ACT>(v[qq], fin(acc[g + NGA][qq], g + NGA, r0 + qq), a);
            else if constexpr (ACT == kActRelu2) v[qq] = fused_relu2(v[qq]);
          }
          *reinterpret_cast<u32x2_t*>(a.C + (int64_t)s * a.ldc + tile_of(strip, g) * kTileN + r0) =
              u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    };
    auto compute = [&](int u) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < NG; ++g)
          acc[g] = mfma(dequant8<QT>(rq[u][g][i], rs[u][g].s(i, lane), rs[u][g].m(i, lane)), rx[u][i], acc[g]);
      if (++cs == L) {
        finish(cq);
        cs = 0;
        ++cq;
      }
    };

    enter(0);
#pragma unroll
    for (int u = 0; u < D; ++u) issue(u);
    const int total = wn * L;
    for (int j0 = 0; j0 < total; j0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        if (j0 + u < total) {
          compute(u);
          issue(u);
        }
      }
    }
    if constexpr (CMB) {
      if (w == 0) combine_all(wn);
    }
  }
}

template <int QT, bool BIAS, int NG, int ACT, int FA, bool CMB>
static int launch_stream_ng(const GemmArgs& a, int ks, int grid, hipStream_t st) {
  switch (ks) {
    case 1: hipLaunchKernelGGL((gemm_stream_kernel<QT, BIAS, NG, 1, ACT, FA, CMB>), dim3(grid), dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((gemm_stream_kernel<QT, BIAS, NG, 2, ACT, FA, CMB>), dim3(grid), dim3(128), 0, st, a); break;
    case 4: hipLaunchKernelGGL((gemm_stream_kernel<QT, BIAS, NG, 4, ACT, FA, CMB>), dim3(grid), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((gemm_stream_kernel<QT, BIAS, NG, 8, ACT, FA, CMB>), dim3(grid), dim3(512), 0, st, a); break;
    default: return fail(MOE_EINVAL, "moe_w4a16_gemm: ksplit=%d (1, 2, 4 or 8)", ks);
  }
  return check_launch("moe_w4a16_gemm (decode stream)");
}

template <int QT, bool BIAS, int ACT, int FA, bool CMB = false>
static int launch_stream_b(const GemmArgs& a, const moe_gemm_config& c, int grid, hipStream_t st) {
  if constexpr (!act_paired<ACT>()) {
    if (c.ng == 1) return launch_stream_ng<QT, BIAS, 1, ACT, FA, CMB>(a, c.ksplit, grid, st);
  }
  switch (c.ng) {
    case 2: return launch_stream_ng<QT, BIAS, 2, ACT, FA, CMB>(a, c.ksplit, grid, st);
    case 4: return launch_stream_ng<QT, BIAS, 4, ACT, FA, CMB>(a, c.ksplit, grid, st);
    default: return fail(MOE_EINVAL, "moe_w4a16_gemm: decode ng=%d (1, 2 or 4; 2 or 4 with a fused gated activation)", c.ng);
  }
}

// the fused align exists for the gate/up GEMM with its activation (the first GEMM of the layer)
template <int QT, bool BIAS, int ACT>
static int launch_stream_fa(const GemmArgs& a, const moe_gemm_config& c, int grid, hipStream_t st) {
  if constexpr (ACT == kActNone) {
    if (a.topk_ids) return fail(MOE_EUNSUPPORTED, "moe_w4a16_gemm: the fused align needs a fused activation");
    return a.cmb_out ? launch_stream_b<QT, BIAS, ACT, 0, true>(a, c, grid, st)
                     : launch_stream_b<QT, BIAS, ACT, 0>(a, c, grid, st);
  } else {
    // (the fused align's second 64-slot batch only when the slots need it: a kernel of its own)
    if (!a.topk_ids) return launch_stream_b<QT, BIAS, ACT, 0>(a, c, grid, st);
    return a.numel > 64 ? launch_stream_b<QT, BIAS, ACT, 2>(a, c, grid, st)
                        : launch_stream_b<QT, BIAS, ACT, 1>(a, c, grid, st);
  }
}

// Persistent grid: about 8 waves per CU and never more workgroups than items, but at least
// enough that no workgroup gets more than kWin items.
template <int QT>
int launch_gemm_stream(bool bias, int act, const GemmArgs& a, const moe_gemm_config& c, int cap_blocks,
                       int num_cus, hipStream_t st) {
  const int NT = a.N / kTileN, KT = a.K / kTileK;
  moe_gemm_config cc = c;  // every wave needs at least one k-tile: ksplit is capped at K/64
  while (cc.ksplit > 1 && cc.ksplit > KT) cc.ksplit /= 2;
  const int nta = act_paired(act) ? NT / 2 : NT, nga = act_paired(act) ? c.ng / 2 : c.ng;
  const int ns = (nta + nga - 1) / std::max(nga, 1);
  const int64_t max_items = (int64_t)cap_blocks * ns;
  const int64_t want = (int64_t)num_cus * std::max(1, 8 / std::max(cc.ksplit, 1));
  const int64_t grid64 = std::max<int64_t>({1, std::min<int64_t>(max_items, want), (max_items + kWin - 1) / kWin});
  if (grid64 >= (1ll << 31)) return fail(MOE_EUNSUPPORTED, "moe_w4a16_gemm: decode grid too large");
  const int grid = (int)grid64;
  switch (act) {
    case kActNone:
      return bias ? launch_stream_fa<QT, true, kActNone>(a, cc, grid, st) : launch_stream_fa<QT, false, kActNone>(a, cc, grid, st);
    case kActSilu:
      return bias ? launch_stream_fa<QT, true, kActSilu>(a, cc, grid, st) : launch_stream_fa<QT, false, kActSilu>(a, cc, grid, st);
    case kActRelu2:
      return bias ? launch_stream_fa<QT, true, kActRelu2>(a, cc, grid, st) : launch_stream_fa<QT, false, kActRelu2>(a, cc, grid, st);
    default:
      return bias ? launch_stream_fa<QT, true, kActSwiglu>(a, cc, grid, st) : launch_stream_fa<QT, false, kActSwiglu>(a, cc, grid, st);
  }
}

}  // namespace moe
