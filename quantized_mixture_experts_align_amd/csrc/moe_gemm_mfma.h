// gemm_mfma: grouped W4A16 GEMM for align blocks of 16/32/64/128 slots (prefill batches).
//
// Workgroup = 4 waves over one align block (16*MG slots of one expert) x 4*NG 16-row weight
// tiles; wave w owns tiles w*NG .. w*NG+NG-1 and all MG 16-slot groups, so every dequantised
// weight fragment feeds MG v_mfma_f32_16x16x32_bf16 (weights = A operand, rows = output
// features; activations = B operand, columns = slots).
//
// Pipeline over K in steps of 64 columns, kStages deep, every operand through LDS:
//   * each stage holds the step's activations (in B-operand order: contiguous ds_read_b128
//     per lane), the wave's NG weight tiles (512 B each, ds_read_b64 per lane) and their group
//     scales, all written by global_load_lds (direct global -> LDS, no register staging);
//   * step kt + kStages - 1 is issued when step kt starts; rows of padding slots read row 0
//     of A (those MFMA columns are never stored);
//   * one barrier per step: at its end each wave waits until its loads of the next step have
//     landed (s_waitcnt vmcnt(n), n = its loads of the steps after that: every load is one
//     instruction, so the count is exact), then all waves meet at s_barrier.
// With ACT (fused gate/up epilogue) the wave's NG tiles are NG/2 gate tiles and the matching up
// tiles I/16 tiles further down, so each lane holds gate and up of the same (slot, column).
#pragma once

#include <type_traits>

#include "moe_gemm_common.h"

namespace moe {

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt[3:0] and
// vmcnt[5:4] at bits 15:14; expcnt and lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Pipeline depth.  Two stages (double buffering) for blocks of 32 slots and more: measured on
// the prefill shapes, three or four are slower (NVFP4 Zipf M=4096 gate/up 1323 -> 1351 us, MXFP4
// M=2048 343 -> 356 us, int4 M=2304 21.2 -> 23.3 us): the smaller LDS footprint lets more
// workgroups share a CU, and those kernels are not limited by the weight stream's latency.
// Three for 16-slot blocks (the decode MFMA configuration), whose few workgroups per CU stream
// weights with little arithmetic in between, so that the bytes in flight set the rate: NVFP4
// slice M=64 layer 170 -> 162 us cold, its down GEMM 50.1 -> 47.6 us (four stages no better).
template <int MG>
constexpr int stages_for() { return MG == 1 ? 3 : 2; }

// Wait until at most n (0..15) of this wave's vector-memory loads are outstanding: s_waitcnt takes
// its count as an immediate, so a wave-uniform run-time count goes through a switch.
__device__ __forceinline__ void wait_vm_upto(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    case 8: wait_vm<8>(); break;
    case 9: wait_vm<9>(); break;
    case 10: wait_vm<10>(); break;
    case 11: wait_vm<11>(); break;
    case 12: wait_vm<12>(); break;
    case 13: wait_vm<13>(); break;
    case 14: wait_vm<14>(); break;
    case 15: wait_vm<15>(); break;
    default: wait_vm<0>(); break;
  }
}

// Slot groups (a divisor of MG) whose outputs the epilogue stages at once: as many as the four
// waves' regions of `per_group` bytes each fit into the pipeline's LDS.
constexpr int epilogue_groups(int MG, int per_group, int lds) {
  int c = MG;
  while (c > 1 && c * per_group > lds) c /= 2;
  return c;
}

// All waves meet.  The wave's own LDS reads of the previous step are waited for first
// (lgkmcnt(0)), so the global->LDS loads issued right after the barrier into that step's stage
// can never overtake them, whatever the compiler schedules before the barrier.
__device__ __forceinline__ void block_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Direct global -> LDS load of BYTES (4 or 16) per lane: lane l's data lands at LDS address
// lds + l*BYTES.
// The address is a wave-uniform 64-bit base in scalar registers + the lane's 32-bit byte offset,
// so a step's address update is scalar work and the per-lane offsets never change.  (No
// instruction offset: for these loads it would move the LDS destination too.)
// Written as inline assembly so that the compiler's own wait insertion, which cannot tell which
// LDS bytes such a load writes, does not add a full vmcnt(0) before every LDS read; the waits
// for these loads are the explicit wait_vm<> calls.  (m0 holds the LDS address; one wait state
// is required between writing m0 and the load.)
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 ::"s"(m0), "v"(voff), "s"(sbase) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 ::"s"(m0), "v"(voff), "s"(sbase) : "memory", "m0");
}

// A pointer that is the same in every lane, held in scalar registers.
__device__ __forceinline__ const uint8_t* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void grouped_block(int nblk, int gm_max, int& mb, int& nb) {
  xcd_grouped_block((int)gridDim.x, (int)blockIdx.x, nblk, gm_max, mb, nb);
}

template <int QT, bool BIAS, int MG, int NG, int ACT>
// (at least two waves per SIMD: the 128-slot, 4-tile variants sit at the 256-register limit,
// and one register more would halve their occupancy)
__global__ __launch_bounds__(256, 2) void gemm_mfma_kernel(GemmArgs a) {
  static_assert(!act_paired<ACT>() || NG % 2 == 0, "the fused gated epilogue pairs gate and up tiles");
  constexpr int NGA = act_paired<ACT>() ? NG / 2 : NG;     // tiles per wave in the assigned range
  constexpr int BM = 16 * MG;
  constexpr int FRAGS = 2 * MG * 64;                      // 16-B activation fragments per step
  constexpr int XL = FRAGS >= 256 ? FRAGS / 256 : 1;      // fragment loads per thread and step
  constexpr int XWAVES = FRAGS >= 256 ? 4 : FRAGS / 64;   // waves that load activations
  constexpr int SROW = TileScale<QT>::kRowBytes;          // scale bytes per tile row
  constexpr int SLANES = 16 * SROW / 4;                    // lanes loading a tile's scales (dwords)
  constexpr int XB = FRAGS * 16;                           // stage layout: activations,
  constexpr int WB = 4 * NG * kTileBytes;                  //   weight tiles of the 4 waves,
  constexpr int SB = 4 * NG * 64;                          //   scales (64-B slot per tile)
  constexpr int kStages = stages_for<MG>();
  constexpr int STAGE = XB + WB + SB;
  constexpr int NWD = (NG + 1) / 2;                        // weight loads per wave and step
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * STAGE];
  __shared__ int s_crow[BM];
  auto stage_ptr = [&](int stage) -> uint8_t* { return smem + stage * STAGE; };
  // the LDS address of smem as a 32-bit integer, so that the DMA destinations are plain scalar
  // sums (a generic pointer converted per load costs a null test and two registers per address)
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  const int NT = a.N / kTileN, KT = a.K / kTileK;
  const int NTA = act_paired<ACT>() ? NT / 2 : NT;          // tiles to assign (gate tiles if fused)
  const int nblk = (NTA + 4 * NGA - 1) / (4 * NGA);
  int mb, nb;
  grouped_block(nblk, a.group_m, mb, nb);
  {
    // with a block schedule, position mb of the launch takes the block the schedule names there
    // (read together with the live length: the schedule has an entry for every position)
    const int ntpp = *a.ntpp;
    if (a.border) {
      const int q = mb;
      mb = a.border[q];
      if (q * BM >= ntpp || mb < 0 || mb >= ntpp / BM) return;  // (no product of an untrusted entry)
    } else if (mb * BM >= ntpp) {
      return;
    }
  }
  const int e = a.eids[mb];
  if (e < 0 || e >= a.E) return;
  // the wave index is uniform: keep it (and every LDS address derived from it) in scalar registers
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  if (tid < BM) {
    const int s = a.sorted[(int64_t)mb * BM + tid];
    s_crow[tid] = (s >= 0 && s < a.numel) ? s : -1;
  }
  __syncthreads();
  // Live 16-slot groups of this block: up to the group of its last live row.  An expert's slots
  // fill its blocks from the front, so only its last block has padding, and there the MFMAs of
  // the all-padding groups are skipped: the tail of each expert runs as a 16/32/.../112-slot
  // tile, chosen here from the expert's row count (results are the same bit for bit).
  int lg;
  {
    const uint64_t m0 = __ballot(lane < BM && s_crow[lane < BM ? lane : 0] >= 0);
    const uint64_t m1 = BM > 64 ? __ballot(s_crow[BM > 64 ? 64 + lane : 0] >= 0) : 0ull;
    const int last = m1 ? 127 - __clzll((long long)m1) : (m0 ? 63 - __clzll((long long)m0) : -1);
    lg = __builtin_amdgcn_readfirstlane((last + 16) >> 4);
  }
  if (lg == 0) return;  // (uniform over the workgroup: no barrier follows for anyone)

  // activation fragment f = l*256 + tid -> k-step i, m-group g, MFMA lane fl: row g*16 + fl%16,
  // columns 32 i + 8 (fl/16) + 0..7 of the step; stage slot f (wave-contiguous for the DMA)
  const bool xwave = w < XWAVES;
  const uint8_t* xbase = uniform_ptr(a.A);
  uint32_t xoff[XL];  // byte offsets from A (the host checks that A spans less than 4 GiB)
#pragma unroll
  for (int l = 0; l < XL; ++l) {
    const int f = l * 256 + tid;
    const int fl = f & 63, g = (f >> 6) % MG, i = (f >> 6) / MG;
    const int row = xwave ? s_crow[g * 16 + (fl & 15)] : -1;
    xoff[l] = (uint32_t)(((int64_t)(row >= 0 ? row / a.top_k : 0) * a.lda + 32 * i + 8 * (fl >> 4)) * 2);
  }
  // weights: NG consecutive 16-row tiles of this wave (clamped at the N edge, not stored)
  int ntile[NG];
  bool nok[NG];
  const uint8_t* wbase[NG];
  const uint8_t* sbase[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g < NGA) {
      const int t = nb * 4 * NGA + w * NGA + g;
      nok[g] = t < NTA;
      ntile[g] = nok[g] ? t : NTA - 1;
    } else {  // up tile of gate tile g - NGA
      nok[g] = nok[g - NGA];
      ntile[g] = ntile[g - NGA] + NTA;
    }
    const int64_t tile0 = ((int64_t)e * NT + ntile[g]) * KT;
    wbase[g] = uniform_ptr(a.codes + tile0 * kTileBytes);
    sbase[g] = uniform_ptr(a.scales + ((int64_t)e * NT + ntile[g]) * (pair_grouped(QT) ? KT / 2 : KT) *
                                          scale_step_bytes(QT));
  }
  // One 16-byte-per-lane load fills two weight tiles of the wave (lanes 0-31 the 512 bytes of tile
  // 2p, lanes 32-63 those of tile 2p+1, through their offset from tile 2p's base; with NG = 1
  // lanes 32-63 stay idle), and one load brings the group scales of all NG tiles (lanes
  // 16g .. 16g + SLANES - 1 those of tile g).  The bytes land where the tiles' LDS slots are
  // contiguous: weights (w*NG + g) * 512, scales (w*NG + g) * 64.  Tile bases never decrease with
  // g, so every offset is a non-negative distance inside one projection's buffer.
  uint32_t woff[NWD];
#pragma unroll
  for (int p = 0; p < NWD; ++p) {
    const uint32_t d = 2 * p + 1 < NG ? (uint32_t)(wbase[2 * p + 1] - wbase[2 * p]) : 0u;
    woff[p] = lane < 32 ? (uint32_t)lane * 16 : d + (uint32_t)(lane - 32) * 16;
  }
  const int sg = lane >> 4, sr = lane & 15;
  const bool s_act = sg < NG && sr < SLANES;
  uint32_t sdist = 0;
#pragma unroll
  for (int g = 1; g < NG; ++g)
    if (sg == g) sdist = (uint32_t)(sbase[g] - sbase[0]);
  const uint32_t soffl = sdist + (uint32_t)sr * 4;
  auto issue = [&](int kt, int stage) {
    const uint32_t st = smem_lds + (uint32_t)(stage * STAGE);
    if (xwave) {
#pragma unroll
      for (int l = 0; l < XL; ++l) {
        // an all-padding 16-slot group's activations are never read (its MFMAs are skipped):
        // not loaded (nload counts what is)
        if (MG > 1 && ((4 * l + w) % MG) >= lg) continue;
        dma_to_lds<16>(xbase + kt * (kTileK * 2), xoff[l], st + (uint32_t)(l * 256 + w * 64) * 16);
      }
    }
#pragma unroll
    for (int p = 0; p < NWD; ++p) {
      const uint32_t wt = st + (uint32_t)(XB + (w * NG + 2 * p) * kTileBytes);
      if (NG > 1 || lane < 32) dma_to_lds<16>(wbase[2 * p] + (int64_t)kt * kTileBytes, woff[p], wt);
    }
    const int64_t soff = (int64_t)(pair_grouped(QT) ? kt >> 1 : kt) * scale_step_bytes(QT);
    if (s_act) dma_to_lds<4>(sbase[0] + soff, soffl, st + (uint32_t)(XB + WB + (w * NG) * 64));
  };

  f32x4_t acc[NG][MG];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int h = 0; h < MG; ++h) acc[g][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // this wave's codes and group scales of one step, from its stage
  auto read_tiles = [&](const uint8_t* st, u32x2_t* wq, TileScale<QT>* sc) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      wq[g] = reinterpret_cast<const u32x2_t*>(st + XB + (w * NG + g) * kTileBytes)[lane];
      const uint8_t* sb = st + XB + WB + (w * NG + g) * 64 + (lane & 15) * SROW;
      sc[g].raw = SROW == 4 ? *reinterpret_cast<const uint32_t*>(sb) : *reinterpret_cast<const uint16_t*>(sb);
    }
  };

  // This wave's loads per step (each load is one instruction whatever its lane mask, and every
  // one of them is issued with lane 0 active): its activation fragments of the live 16-slot
  // groups, its weight loads and its scale load.
  int nload = NWD + 1;
  if (xwave) {
#pragma unroll
    for (int l = 0; l < XL; ++l)
      if (!(MG > 1 && ((4 * l + w) % MG) >= lg)) ++nload;
  }
  // At the end of step kt (or of the prologue, "step -1") each wave waits until its loads of step
  // kt + 1 have landed -- only those of the steps after it may still be in flight -- and all waves
  // meet at the barrier: step kt + 1's operands are then in LDS for everyone, and everyone is done
  // with step kt's stage, which the loads issued at the start of step kt + 1 overwrite.
  auto wait_next = [&](int kt) {
    if constexpr (kStages == 2) {
      wait_vm<0>();  // (no later step's loads have been issued yet)
    } else {
      const int later = max(0, min(kt + kStages - 1, KT - 1) - (kt + 1));
      wait_vm_upto(later * nload);
    }
    block_barrier();
  };
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < KT) issue(s, s);
  wait_next(-1);

  // One step's dequantisation and MFMAs.  With PARTIAL (an expert's last block), the 16-slot
  // groups from lg on are all padding and their MFMAs are skipped; full blocks run without those
  // branches.
  auto compute = [&](auto partial, const uint8_t* st) {
    constexpr bool PARTIAL = decltype(partial)::value;
    const u32x4_t* xs = reinterpret_cast<const u32x4_t*>(st);
    u32x2_t wq[NG];
    TileScale<QT> sc[NG];
    read_tiles(st, wq, sc);
    if constexpr (PARTIAL || MG < NG) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        u32x4_t af[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) af[g] = dequant8<QT>(wq[g][i], sc[g].s(i, lane), sc[g].m(i, lane));
#pragma unroll
        for (int h = 0; h < MG; ++h) {
          if constexpr (PARTIAL) {
            if (h >= lg) break;
          }
          const u32x4_t bf = xs[(i * MG + h) * 64 + lane];
#pragma unroll
          for (int g = 0; g < NG; ++g) acc[g][h] = mfma(af[g], bf, acc[g][h]);
        }
      }
    } else {
      // full block: the second substep's dequantisation is computed tile by tile between the
      // first substep's MFMA groups (scheduling barriers keep each chunk in place; left to itself
      // the compiler issues all of it after the MFMA run), so one wave keeps VALU and matrix core
      // busy together; the activation fragment of the next group is read one chunk ahead.
      // Measured: NVFP4 Zipf M=4096 gate/up GEMM 1436 -> 1398 us, M=1024 layer 736 -> 709 us.
      u32x4_t a0[NG], a1[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) a0[g] = dequant8<QT>(wq[g][0], sc[g].s(0, lane), sc[g].m(0, lane));
      u32x4_t bf = xs[lane];
#pragma unroll
      for (int h = 0; h < MG; ++h) {
        const u32x4_t bn = xs[(h + 1) * 64 + lane];   // (h + 1 = MG: the first of substep 1)
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g][h] = mfma(a0[g], bf, acc[g][h]);
        if (h < NG) a1[h] = dequant8<QT>(wq[h][1], sc[h].s(1, lane), sc[h].m(1, lane));
        bf = bn;
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int h = 0; h < MG; ++h) {
        const u32x4_t bn = h + 1 < MG ? xs[(MG + h + 1) * 64 + lane] : bf;
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g][h] = mfma(a1[g], bf, acc[g][h]);
        bf = bn;
      }
    }
  };

  auto step = [&](auto partial, int kt, int u) {
    if (kt + kStages - 1 < KT) issue(kt + kStages - 1, (u + kStages - 1) % kStages);
    compute(partial, stage_ptr(u));
    wait_next(kt);
  };
  // whole rounds of kStages steps (stage index = compile-time constant), then the remaining steps;
  // no early exit inside the unrolled round, which would make the accumulators change registers
  auto k_loop = [&](auto partial) {
    int kt0 = 0;
    for (; kt0 + kStages <= KT; kt0 += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) step(partial, kt0 + u, u);
    }
#pragma unroll
    for (int u = 0; u < kStages - 1; ++u)
      if (kt0 + u < KT) step(partial, kt0 + u, u);
  };
  if (MG == 1 || lg == MG) k_loop(std::false_type{});
  else k_loop(std::true_type{});

  // epilogue: lane holds D[n = 4 (lane/16) + q][m = lane % 16] of each (n-tile, m-group)
  float gsv = 1.f;
  if constexpr (QT == MOE_Q_NVFP4_G16) gsv = a.gs[e];
  float bv[NG][4];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int n0 = ntile[g] * kTileN + 4 * (lane >> 4);
    bv[g][0] = bv[g][1] = bv[g][2] = bv[g][3] = 0.f;
    if constexpr (BIAS) {
      const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(a.bias + (int64_t)e * a.N + n0);
      bv[g][0] = bf16_lo(bb[0]); bv[g][1] = bf16_hi(bb[0]); bv[g][2] = bf16_lo(bb[1]); bv[g][3] = bf16_hi(bb[1]);
    }
  }
  // the output values of tile g, slot group h, column 4 (lane/16) + q: scale, bias, activation,
  // packed to bf16
  auto out4 = [&](int g, int h) {
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[q] = acc[g][h][q] * gsv + bv[g][q];
      if constexpr (act_paired<ACT>()) o[q] = fused_act<ACT>(o[q], acc[g + NGA][h][q] * gsv + bv[g + NGA][q], a);
      else if constexpr (ACT == kActRelu2) o[q] = fused_relu2(o[q]);
    }
    return u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
  };
  constexpr int COLS = 16 * NGA;         // output columns of the wave (consecutive tiles)
  constexpr int PITCH = 2 * COLS + 16;   // LDS bytes per staged slot row (padded against bank conflicts)
  constexpr int CH = epilogue_groups(MG, 4 * 16 * PITCH, kStages * STAGE);
  if (((uintptr_t)a.C & 15) == 0 && (a.ldc & 7) == 0) {
    // Staged through LDS, idle once every wave has passed the last step's barrier: each wave
    // writes CH slot groups of its tiles to its own region, then stores them as 16 bytes per lane
    // with the lanes of a slot row on consecutive columns, so that an instruction covers whole
    // row segments of the wave's 16 x NGA columns (unstaged, each writes 16 rows x 32 bytes).
    // Values and rounding are those of the unstaged stores.  Measured, same box, alternating:
    // NVFP4 Zipf down GEMM 780 -> 743 us at M = 4096 and 237 -> 223 us at M = 1024, MXFP4 M = 2048
    // down 195 -> 189 us, gate/up GEMMs and decode within noise (without any stores, timing only,
    // the down GEMM was 9% faster).
    uint8_t* wl = smem + w * (CH * 16 * PITCH);
    constexpr int CHUNKS = COLS / 8;      // 16-byte chunks per row
    constexpr int RPI = 64 / CHUNKS;      // rows per store instruction
    const int t0 = nb * 4 * NGA + w * NGA;  // the wave's first tile (unclamped)
    const int j = lane % CHUNKS;
    const bool col_ok = t0 + j / 2 < NTA;   // (chunk j lies in tile t0 + j/2)
    uint16_t* cbase = a.C + (int64_t)t0 * kTileN + 8 * j;
    // (only the live slot groups, h < lg: the rest of an expert's last block is padding)
#pragma unroll
    for (int h0 = 0; h0 < MG; h0 += CH) {
      if (h0 >= lg) break;
#pragma unroll
      for (int g = 0; g < NGA; ++g)
#pragma unroll
        for (int c = 0; c < CH; ++c)
          if (h0 + c < lg)
            *reinterpret_cast<u32x2_t*>(wl + ((c * 16 + (lane & 15)) * PITCH + (g * 16 + 4 * (lane >> 4)) * 2)) =
                out4(g, h0 + c);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int r0 = 0; r0 < CH * 16; r0 += RPI) {
        if (r0 >= (lg - h0) * 16) break;
        const int sl = r0 + lane / CHUNKS;
        if (RPI <= CH * 16 || sl < CH * 16) {
          const int row = s_crow[h0 * 16 + sl];
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wl + sl * PITCH + 16 * j);
          if (row >= 0 && col_ok) *reinterpret_cast<u32x4_t*>(cbase + (int64_t)row * a.ldc) = v;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  } else {
#pragma unroll
    for (int g = 0; g < NGA; ++g) {
      if (!nok[g]) continue;
      const int n0 = ntile[g] * kTileN + 4 * (lane >> 4);
#pragma unroll
      for (int h = 0; h < MG; ++h) {
        const int row = s_crow[h * 16 + (lane & 15)];
        if (row < 0) continue;
        *reinterpret_cast<u32x2_t*>(a.C + (int64_t)row * a.ldc + n0) = out4(g, h);
      }
    }
  }
}

template <int QT, bool BIAS, int MG, int ACT>
static int launch_mg(const GemmArgs& a, int ng, int blocks, hipStream_t st) {
  const int NT = a.N / kTileN;
  const int nta = act_paired<ACT>() ? NT / 2 : NT, nga = act_paired<ACT>() ? ng / 2 : ng;
  const int nblk = (nta + 4 * nga - 1) / (4 * nga);
  const dim3 grid((unsigned)((int64_t)nblk * blocks));
  if constexpr (!act_paired<ACT>()) {
    if (ng == 1) {
      hipLaunchKernelGGL((gemm_mfma_kernel<QT, BIAS, MG, 1, ACT>), grid, dim3(256), 0, st, a);
      return check_launch("moe_w4a16_gemm (mfma)");
    }
  }
  switch (ng) {
    case 2: hipLaunchKernelGGL((gemm_mfma_kernel<QT, BIAS, MG, 2, ACT>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((gemm_mfma_kernel<QT, BIAS, MG, 4, ACT>), grid, dim3(256), 0, st, a); break;
    default:
      return fail(MOE_EINVAL, "moe_w4a16_gemm: ng=%d (1, 2 or 4; 2 or 4 with a fused gated activation)", ng);
  }
  return check_launch("moe_w4a16_gemm (mfma)");
}

template <int QT, bool BIAS, int ACT>
static int launch_mfma_b(const GemmArgs& a, int ng, int blocks, hipStream_t st) {
  switch (a.block_m) {
    case 16: return launch_mg<QT, BIAS, 1, ACT>(a, ng, blocks, st);
    case 32: return launch_mg<QT, BIAS, 2, ACT>(a, ng, blocks, st);
    case 64: return launch_mg<QT, BIAS, 4, ACT>(a, ng, blocks, st);
    case 128: return launch_mg<QT, BIAS, 8, ACT>(a, ng, blocks, st);
    default:
      return fail(MOE_EUNSUPPORTED, "moe_w4a16_gemm: MFMA kernel needs block_m 16/32/64/128, got %d",
                  a.block_m);
  }
}

// Resident workgroups per CU of one kernel variant on the current device, as the HIP occupancy
// API computes them from its registers and LDS (0 when the runtime does not answer).
template <int QT, bool BIAS, int MG, int NG, int ACT>
static int resident_of() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&gemm_mfma_kernel<QT, BIAS, MG, NG, ACT>), 256, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

template <int QT, bool BIAS, int MG, int ACT>
static void resident_mg(int* r) {
  if constexpr (act_paired<ACT>()) r[0] = 0;
  else r[0] = resident_of<QT, BIAS, MG, 1, ACT>();
  r[1] = resident_of<QT, BIAS, MG, 2, ACT>();
  r[2] = resident_of<QT, BIAS, MG, 4, ACT>();
}

template <int QT, bool BIAS, int ACT>
static int residency_b(int block_m, int* r) {
  switch (block_m) {
    case 16: resident_mg<QT, BIAS, 1, ACT>(r); return 0;
    case 32: resident_mg<QT, BIAS, 2, ACT>(r); return 0;
    case 64: resident_mg<QT, BIAS, 4, ACT>(r); return 0;
    case 128: resident_mg<QT, BIAS, 8, ACT>(r); return 0;
    default: return -1;
  }
}

// r[0..2]: resident workgroups per CU at ng = 1, 2, 4 (the SiLU variant stands for both gated
// activations, the plain one for the others; their register use is within a few of each other).
template <int QT>
int mfma_residency(bool bias, bool gated, int block_m, int* r) {
  if (gated) return bias ? residency_b<QT, true, kActSilu>(block_m, r) : residency_b<QT, false, kActSilu>(block_m, r);
  return bias ? residency_b<QT, true, kActNone>(block_m, r) : residency_b<QT, false, kActNone>(block_m, r);
}

template <int QT>
int launch_gemm_mfma(bool bias, int act, const GemmArgs& a, const moe_gemm_config& c, int cap_blocks,
                     hipStream_t st) {
  switch (act) {
    case kActNone:
      return bias ? launch_mfma_b<QT, true, kActNone>(a, c.ng, cap_blocks, st)
                  : launch_mfma_b<QT, false, kActNone>(a, c.ng, cap_blocks, st);
    case kActSilu:
      return bias ? launch_mfma_b<QT, true, kActSilu>(a, c.ng, cap_blocks, st)
                  : launch_mfma_b<QT, false, kActSilu>(a, c.ng, cap_blocks, st);
    case kActRelu2:
      return bias ? launch_mfma_b<QT, true, kActRelu2>(a, c.ng, cap_blocks, st)
                  : launch_mfma_b<QT, false, kActRelu2>(a, c.ng, cap_blocks, st);
    default:
      return bias ? launch_mfma_b<QT, true, kActSwiglu>(a, c.ng, cap_blocks, st)
                  : launch_mfma_b<QT, false, kActSwiglu>(a, c.ng, cap_blocks, st);
  }
}

}  // namespace moe
