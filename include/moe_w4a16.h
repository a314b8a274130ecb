/*
 * moe_w4a16.h -- C ABI of the MI355X (gfx950) W4A16 mixture-of-experts expert layer.
 *
 * The layer, for one GPU's slice of experts [expert_start, expert_start + n_local):
 *
 *   moe_align        route the top-k (token, slot) assignments to local experts and
 *                    sort them into per-expert blocks of block_m rows
 *   moe_w4a16_gemm   gate/up projection: h[slot] = dequant(W13[e]) x[slot / top_k] (+ b13[e])
 *   moe_act          a = silu(gate) * up, or GPT-OSS gate * sigmoid(alpha * gate) * (up + 1)
 *   moe_w4a16_gemm   down projection:    y[slot] = dequant(W2[e]) a[slot] (+ b2[e])
 *   moe_combine      out[t] = sum over live slots of g * y, optionally after the
 *                    weight-first post-expert RMSNorm with weight bf16(1 + w)
 *
 * and, for the W4AFP8 variant of the expert path, moe_fp8_requant: float8 activations
 * quantised per token and group re-expressed against one per-tensor scale.
 *
 * Sources.  The steps and their arguments follow the pages the method is described on:
 * the Muse Spark NVFP4 experiment "013-moe-middle-tiles.py" (bishal.us open-kernel-challenge):
 * Inputs / Weights / Config, prepare and kernel_fn (expert_map, moe_align_block_size, two
 * moe_wna16_marlin_gemm calls, silu_and_mul, _expert_norm_factors / _expert_norm_sum); the
 * "sglang PR 31552" summary (Marlin MoE W4A16: kIsEP / kHasBias, the per-expert reference loop
 * with biases); the "sglang PR 28231" summary (MXFP4 on Marlin: gate/up de-interleave, tile
 * padding, swiglu_gpt_oss_sigmoid_alpha_contiguous).
 *
 * Conventions (every function):
 *   - Pointers marked "device" are device memory owned by the caller; host structs and sizes
 *     are passed by value or by host pointer.  Nothing is allocated or freed, nothing is
 *     synchronised: work is enqueued on `stream` (0 = the null stream) and returns at once.
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major, rows contiguous unless a
 *     leading dimension is given.
 *   - Return 0 (MOE_OK) or a negative moe_status.  Arguments are validated on the host before
 *     anything is launched; on error nothing is launched and moe_last_error() describes why.
 *   - Device data is never trusted to be in range: expert ids outside the local range are
 *     dropped, sorted ids at or past `numel` are padding and are skipped.
 *   - Calls are thread-safe (no global mutable state besides the thread-local error text).
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* bad argument: null pointer, negative or inconsistent size */
  MOE_EUNSUPPORTED = -2,  /* valid but not implemented (shape not a tile multiple, ...) */
  MOE_ESIZE = -3,         /* caller buffer too small */
  MOE_EHIP = -4           /* a HIP runtime call failed (launch error, no device) */
} moe_status;

typedef enum {
  MOE_Q_INT4_G128 = 0,    /* uint4b8: nibble u means u - 8; bf16 scale per 128 along K       */
  MOE_Q_NVFP4_G16 = 1,    /* E2M1 codes; float8 e4m3fn scale per 16 along K; fp32 global/expert */
  MOE_Q_MXFP4_G32 = 2,    /* E2M1 codes; E8M0 scale per 32 along K                            */
  MOE_Q_INT4ZP_G128 = 3,  /* asymmetric int4: unsigned nibble u, integer zero point z (0..15)
                             and bf16 scale s per 128 along K; the weight is (u - z) * s     */
  MOE_Q_INT4ZPF_G128 = 4, /* asymmetric int4 with float zero points (the Marlin template's
                             is_zp_float case of the "sglang PR 31552" summary): unsigned
                             nibble u, float16 zero point z and bf16 scale s per 128 along K;
                             the weight is (u - z) * s                                       */
  /* (range sentinels, never valid arguments: they make the type's range all of int32, so that
     an unknown value reaches the library's validation and comes back as MOE_EINVAL)          */
  MOE_Q_RANGE_MIN_ = -2147483647 - 1,
  MOE_Q_RANGE_MAX_ = 2147483647
} moe_qtype;

typedef enum {
  MOE_ACT_SILU_MUL = 0,      /* gated: silu(gate) * up                                      */
  MOE_ACT_SWIGLU_ALPHA = 1,  /* gated: min(g,L) * sigmoid(alpha * min(g,L)) * (clamp(u,-L,L) + 1) */
  MOE_ACT_RELU2 = 2,         /* non-gated: relu(h)^2 (the sglang PR 31552 test's activation,
                                is_gated=False; GEMM1 then has I rows, no gate/up halves)  */
  MOE_ACT_RANGE_MIN_ = -2147483647 - 1,  /* range sentinels, as for moe_qtype */
  MOE_ACT_RANGE_MAX_ = 2147483647
} moe_act_kind;

/* ----------------------------------------------------------------------------- errors */

/* Text of the last non-zero return on the calling thread ("" if none).  Owned by the library. */
const char* moe_last_error(void);

/* Library ABI version (incremented on any incompatible change). */
int32_t moe_abi_version(void);

/* ----------------------------------------------------------------------------- align */

/*
 * Sizes of the align outputs for M tokens with top_k slots each:
 *   *sorted_len = number of int32 entries of sorted_token_ids,
 *   *blocks_len = number of int32 entries of expert_ids = *sorted_len / block_m.
 * At most min(n_local, M*top_k) experts are non-empty and each pads by at most block_m - 1,
 * so the padded total never exceeds numel + min(n_local, numel) * (block_m - 1); rounded up
 * to whole blocks.  Pure host function.
 */
int moe_align_capacity(int64_t M, int32_t top_k, int32_t n_local, int32_t block_m,
                       int64_t* sorted_len, int64_t* blocks_len);

/*
 * Route and align (the experiment's expert_map gather + moe_align_block_size).
 *   topk_ids          device int32 [M, top_k], global expert ids
 *   expert_start,
 *   n_local           local experts are [expert_start, expert_start + n_local); 1..512
 *   block_m           rows per block, 1..256
 * Outputs (device, caller-allocated with moe_align_capacity sizes):
 *   sorted_token_ids  int32 [sorted_len] (may be NULL when sorted_len is 0): expert 0's flat slot ids t*top_k+s in ascending order,
 *                     padded with the sentinel numel = M*top_k to a multiple of block_m, then
 *                     expert 1's, ...; empty experts get no block; the rest is the sentinel.
 *   expert_ids        int32 [blocks_len]: local expert of each block, -1 after the last block.
 *   num_tokens_post_padded  int32 [1]: total padded length (a multiple of block_m).
 *   slot_local_ids    int32 [M, top_k] or NULL: local expert of each slot, -1 when the
 *                     assignment is outside the local range (dropped).
 * The result is unique (a stable counting sort), computed by one workgroup without atomics
 * deciding the order.
 */
int moe_align(const int32_t* topk_ids, int64_t M, int32_t top_k, int32_t expert_start,
              int32_t n_local, int32_t block_m, int32_t* sorted_token_ids, int32_t* expert_ids,
              int32_t* num_tokens_post_padded, int32_t* slot_local_ids, hipStream_t stream);

/*
 * moe_align plus a block schedule for the MFMA GEMM (moe_gemm_config.block_order): the same
 * four outputs, bit for bit, and
 *   block_order       device int32 [blocks_len]: entry q < nb (nb = num_tokens_post_padded /
 *                     block_m, the live blocks) is a block index; entries from nb on are -1.
 *                     The live blocks appear once each, ordered by falling 16-slot group count
 *                     ceil(live rows / 16) -- first every block with a full block's count
 *                     (the full blocks and the experts' last blocks that fill as many groups),
 *                     then the experts' shorter last blocks -- and by block index among equal
 *                     counts.
 * Why: a block costs its GEMM workgroups roughly in proportion to its live 16-slot groups (an
 * expert's short last block about half a full one), and the GEMM gives whole align blocks to the
 * eight XCDs in turn.  In align order a regular pattern of full and short blocks can give some XCDs
 * only full blocks (uniform routing: full, short, full, short, ...), and the launch ends on
 * whichever blocks come last.  In falling-cost order the XCDs' shares differ by at most one block
 * and the launch ends on the shortest blocks.  Measured (one MI355X, NVFP4 expert slice with Zipf
 * routing, whole layer): 1024 tokens 718 -> 695 us (down GEMM 231 -> 218 us), 256 tokens 335 ->
 * 326 us, 4096 tokens 2250 -> 2227 us; keeping align order and alternating costly and cheap blocks
 * inside rounds of eight gained less (1024 tokens 712 us).  (The pages give no block scheduler:
 * this is a launch-order choice of this library's GEMM and changes no result.)
 * Errors as moe_align; block_order NULL with blocks_len > 0 is MOE_EINVAL.
 */
int moe_align_sched(const int32_t* topk_ids, int64_t M, int32_t top_k, int32_t expert_start,
                    int32_t n_local, int32_t block_m, int32_t* sorted_token_ids, int32_t* expert_ids,
                    int32_t* num_tokens_post_padded, int32_t* slot_local_ids, int32_t* block_order,
                    hipStream_t stream);

/* ----------------------------------------------------------------------------- weights */

/* prepare flags */
#define MOE_PREP_GATE_UP      0x1u  /* rows are a gate/up pair: N = 2I, gate rows [0, I), up [I, 2I) */
#define MOE_PREP_INTERLEAVED  0x2u  /* with GATE_UP: rows arrive as gate0, up0, gate1, up1, ...   */
#define MOE_PREP_PAD          0x4u  /* zero-pad K (and with GATE_UP each half of N) to a multiple of 64 */
#define MOE_PREP_ACT_ORDER    0x8u  /* int4 formats: act-order grouping (g_idx); the prepared
                                       columns are in group order, desc.perm gives their source */

/* Prepared (device-resident) weights of one projection, filled by moe_w4a16_prepare.  Plain
 * data: it may be copied; the pointers are into the caller's `out` buffer. */
typedef struct moe_weights {
  int32_t qtype;          /* moe_qtype */
  int32_t n_experts;      /* E */
  int32_t N;              /* output rows per expert in the prepared layout (padded)   */
  int32_t K;              /* reduction length in the prepared layout (padded)         */
  int32_t N_logical;      /* rows as given (2I for a gate/up pair)                     */
  int32_t K_logical;
  uint32_t flags;         /* the MOE_PREP_* flags used                                 */
  int32_t reserved;
  const void* codes;      /* tiled 4-bit codes                                         */
  const void* scales;     /* tiled group scales (and zero points)                      */
  const float* global_scale; /* [E] NVFP4 per-expert scale, else NULL                  */
  const uint16_t* bias;   /* bf16 [E, N] or NULL                                       */
  const int32_t* perm;    /* act-order: int32 [E, K]; prepared column j of expert e is input
                             column perm[e * K + j] (moe_permute_cols gathers the activations
                             into this order); NULL without MOE_PREP_ACT_ORDER              */
} moe_weights;

/* Prepared dimensions and the number of bytes moe_w4a16_prepare writes.  Pure host function.
 * Requirements: N % 16 == 0 (N % 32 with GATE_UP) and K % 64 == 0 unless MOE_PREP_PAD is set;
 * K % group == 0 always (group 128 / 16 / 32 by qtype). */
int moe_w4a16_prepared_size(moe_qtype q, int32_t E, int32_t N, int32_t K, uint32_t flags,
                            int32_t has_bias, int32_t* N_out, int32_t* K_out, size_t* bytes);

/*
 * Load-time repack (the experiment's prepare / prepare_moe_nvfp4_layer_for_marlin step, and
 * for GPT-OSS the de-interleave and tile padding of sglang PR 28231).  Untimed.
 *   codes         device uint8 [E, N, K/2], two codes per byte, low nibble = even k
 *   scales        device [E, N, K/g]: bf16 bits (both int4 formats), e4m3fn codes (NVFP4), E8M0
 *                 codes (MXFP4)
 *   global_scale  device fp32 [E] (NVFP4 only, else NULL)
 *   bias          device bf16 [E, N] or NULL (interleaved like the rows when INTERLEAVED)
 *   zeros         MOE_Q_INT4ZP_G128: device uint8 [E, N, K/128], zero points 0..15 (a value above
 *                 15 is an error of the caller and is used modulo 16); MOE_Q_INT4ZPF_G128: device
 *                 uint16 [E, N, K/128], float16 bit patterns; NULL for the other formats
 *   g_idx         device int32 [E, K] with MOE_PREP_ACT_ORDER (int4 formats, K <= 16384), else
 *                 NULL: the group of 128 whose scale (and zero point) input column k uses -- the
 *                 g_idx of the Marlin MoE call in the "sglang PR 31552" summary, the GPTQ
 *                 act-order grouping.  Every group must hold exactly 128 columns; otherwise the
 *                 results are undefined (memory stays in bounds: out-of-range ids are ignored).
 *                 The columns are stored sorted by group (stable), so that the GEMMs see the
 *                 plain grouping, and desc->perm records the order.
 *   out           device buffer of at least `bytes` from moe_w4a16_prepared_size, 256-B aligned
 *   desc          host struct filled with the prepared dims and device pointers into `out`
 * Padded rows/columns get zero weights (zero codes, and zero points equal to the code for the
 * int4 formats), unit scales and zero bias, which leaves the layer's result unchanged
 * (act(0, 0) = 0 for every activation).
 */
int moe_w4a16_prepare(moe_qtype q, const uint8_t* codes, const void* scales,
                      const float* global_scale, const uint16_t* bias, const void* zeros,
                      const int32_t* g_idx, int32_t E, int32_t N, int32_t K, uint32_t flags,
                      void* out, size_t out_bytes, moe_weights* desc, hipStream_t stream);

/*
 * Act-order activation gather: the rows a GEMM on act-order weights reads, with their columns
 * in the prepared (group-sorted) order of the expert each row is routed to:
 *   dst[r, j] = src[r / row_div, perm[e * K + j]],   e = slot_expert[r]
 * for every r < rows with 0 <= e < E; other rows of dst are not written.
 *   src          device bf16 [*, ld_src]: the layer input (row_div = top_k, rows = M * top_k,
 *                one row per slot) or GEMM1's activated output (row_div = 1)
 *   perm         desc.perm of the act-order projection (int32 [E, K])
 *   slot_expert  device int32 [rows]: local expert of each slot (moe_align's slot_local_ids)
 *   dst          device bf16 [rows, ld_dst], the GEMM's A with top_k = 1
 * K % 8 == 0; ld_src, ld_dst >= K; src and dst must not overlap.  Errors: MOE_EINVAL.
 */
int moe_permute_cols(const uint16_t* src, int64_t ld_src, int32_t row_div, const int32_t* perm,
                     int32_t K, int32_t E, const int32_t* slot_expert, int64_t rows, uint16_t* dst,
                     int64_t ld_dst, hipStream_t stream);

/* The post-expert norm's effective weight: out[h] = bf16(1 + w[h]) (round to nearest even),
 * as the experiment's prepare binds it once.  w, out: device bf16 [H]. */
int moe_norm_weight(const uint16_t* w, int32_t H, uint16_t* out, hipStream_t stream);

/* ----------------------------------------------------------------------------- GEMM */

typedef enum {
  MOE_GEMM_AUTO = 0,
  MOE_GEMM_DECODE = 1,    /* block_m <= 16: persistent workgroups over (live block, strip of ng
                             16-row weight tiles), K split over ksplit waves.  gemv_rows = 0:
                             the streaming kernel (one 16-slot MFMA column per tile, one
                             uninterrupted prefetch ring per wave across its items);
                             gemv_rows > 0: dot products for blocks of <= gemv_rows live slots,
                             the MFMA column otherwise                                        */
  MOE_GEMM_MFMA = 2       /* block_m in {16,32,64,128}: 4 waves x ng 16-row tiles x all slots of
                             the block, bf16 MFMA 16x16x32, activations through an LDS ring   */
} moe_gemm_kernel;

/* Launch configuration.  For the MFMA kernel every valid configuration gives the same result bit
 * for bit (the K order of every output is fixed); for the decode kernel a fixed configuration is
 * reproducible run to run, and configurations differ only by fp32 summation order.  AUTO
 * (cfg NULL or kernel 0) picks one from the shapes. */
typedef struct moe_gemm_config {
  int32_t kernel;         /* moe_gemm_kernel                                               */
  int32_t ng;             /* 16-row weight tiles per wave: 1, 2 or 4 (2 or 4 with a fused
                             gated activation: gate and up tiles in pairs; else MOE_EINVAL)   */
  int32_t ksplit;         /* DECODE: waves splitting K in one workgroup: 1, 2, 4 (or 8 when
                             gemv_rows = 0); capped at K/64 by the streaming kernel           */
  int32_t gemv_rows;      /* DECODE: blocks with at most this many live slots use dot
                             products (0..4, and gemv_rows * K * 2 <= 32 KiB)              */
  int32_t group_m;        /* MFMA: align blocks per workgroup group, 0..64 (0 = chosen from
                             the shapes); a group's workgroups run on one XCD, sharing its
                             L2.  Launch order only: results do not depend on it             */
  const int32_t* block_order; /* MFMA: device int32 [blocks_len], the block schedule that
                             moe_align_sched wrote for the same align call, or NULL (blocks
                             in align order).  The workgroups take their align blocks in this
                             order.  Launch order only: results do not depend on it; an entry
                             that names no live block makes its workgroups skip it */
} moe_gemm_config;

/* Host heuristics (pure host functions).  moe_choose_block_m: block_m for the align from the
 * slot count numel = M * top_k, the local experts, the slots expected to be live on this slice
 * (expected_live <= 0: all of them) and the gate/up reduction length K (<= 0: unknown, taken as
 * long).  moe_gemm_choose: the GEMM configuration for projection W; `numel` is the number
 * of slots expected to be live (M * top_k when unknown, or the expected local share of it -- a
 * launch hint only, never a correctness input), num_cus <= 0 means 256. */
int moe_choose_block_m(int64_t numel, int32_t n_local, int64_t expected_live, int32_t K, int32_t* block_m);
int moe_gemm_choose(const moe_weights* W, int64_t numel, int32_t block_m, int32_t num_cus,
                    moe_gemm_config* cfg);

/*
 * Residency of the MFMA GEMM kernel that moe_w4a16_gemm launches for projection W with this
 * block_m (16, 32, 64 or 128): resident[i] = workgroups (of four waves) that fit one compute unit
 * at once with 1, 2 and 4 weight tiles per wave, as the HIP occupancy API computes them on the
 * current device from each kernel variant's register and LDS use.  gated != 0: the variant with a
 * fused gated activation (its resident[0] is 0: it has no one-tile form).  Asked once per device
 * and variant, then cached.  Errors: MOE_EINVAL for bad arguments, MOE_EHIP when no device
 * answers.  This is what moe_gemm_choose weighs the tile counts of the prefill GEMMs with (the
 * occupancy-driven part of the launch choice, [PR31552]'s determine_exec_config role).
 */
int moe_gemm_occupancy(const moe_weights* W, int32_t block_m, int32_t gated, int32_t resident[3]);

/*
 * moe_gemm_choose with the MFMA residency given instead of asked of the device (resident[i] at
 * 1, 2, 4 tiles per wave, as moe_gemm_occupancy returns it).  moe_gemm_choose calls this with the
 * current device's residency (two per CU, the kernels' launch bound, when no device answers).
 * For the prefill block sizes (32 to 128 slots): two tiles per wave; four when the weights stream
 * through long K loops (64-slot blocks with K >= 2048) or the blocks hold 128 slots, the four-tile
 * grid gives every CU a workgroup, and it needs no more rounds of resident workgroups than the
 * two-tile grid; one tile when the two-tile grid has fewer workgroups than CUs.  Pure host function.
 */
int moe_gemm_choose_occ(const moe_weights* W, int64_t numel, int32_t block_m, int32_t num_cus,
                        const int32_t resident[3], moe_gemm_config* cfg);

/*
 * Grouped W4A16 GEMM over the align blocks (moe_wna16_marlin_gemm with mul_topk_weights=False,
 * fp32 accumulation).  For every sorted entry s < numel of block b (expert e = expert_ids[b]):
 *     C[s, n] = bf16( gs[e] * sum_k dequant(W[e])[n, k] * A[s / top_k, k]  (+ bias[e, n]) )
 *   A        device bf16 [a_rows, lda], K = W->K columns read (columns >= K_logical of the
 *            padded part must be zero or finite: their weights are zero)
 *   C        device bf16 [numel, ldc]; only rows of live slots are written, N = W->N columns
 *   sorted_token_ids, expert_ids, num_tokens_post_padded: moe_align outputs for
 *            n_local = W->n_experts and this block_m; `numel` = M * top_k of that align
 *   top_k    A row of entry s is s / top_k (the token); 1 for the down projection
 *   cfg      NULL for AUTO
 * Dequantised weights are rounded to bf16 before the bf16 x bf16 MFMA products (exact for
 * NVFP4 and MXFP4; int4 (u-8)*s is rounded like the Marlin kernel does).
 * Act-order weights (W->perm != NULL) store their columns in group order: A must hold each
 * slot's row with its columns in that order (moe_permute_cols, one row per slot, top_k = 1).
 */
int moe_w4a16_gemm(const uint16_t* A, int64_t a_rows, int32_t lda, uint16_t* C, int32_t ldc,
                   const moe_weights* W, const int32_t* sorted_token_ids,
                   const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                   int64_t numel, int32_t top_k, int32_t block_m, const moe_gemm_config* cfg,
                   hipStream_t stream);

/*
 * GEMM1 with the activation fused into its epilogue (one launch instead of moe_w4a16_gemm +
 * moe_act, and no [numel, 2I] intermediate in memory).  Gated kinds:
 *     out[s, j] = act(gate, up),  gate = bf16(h[s, j]), up = bf16(h[s, I + j])
 * where h is what moe_w4a16_gemm computes for W13 (prepared with MOE_PREP_GATE_UP, N = 2I);
 * cfg->ng must be 2 or 4 (gate/up tile pairs).  MOE_ACT_RELU2: W13 is a plain projection (not
 * MOE_PREP_GATE_UP, N = I) and out[s, j] = relu(bf16(h[s, j]))^2.  The GEMM values are rounded
 * to bf16 exactly as the stored GEMM output would be, so the result equals moe_w4a16_gemm
 * followed by moe_act bit for bit.  out: device bf16 [numel, ldo], ldo >= I, only rows of live
 * slots written.  Other arguments as moe_w4a16_gemm; alpha/limit as moe_act.
 */
int moe_w4a16_gemm_act(moe_act_kind kind, float alpha, float limit, const uint16_t* A, int64_t a_rows,
                       int32_t lda, uint16_t* out, int32_t ldo, const moe_weights* W13,
                       const int32_t* sorted_token_ids, const int32_t* expert_ids,
                       const int32_t* num_tokens_post_padded, int64_t numel, int32_t top_k,
                       int32_t block_m, const moe_gemm_config* cfg, hipStream_t stream);

/*
 * moe_align fused into moe_w4a16_gemm_act, for small batches: the single-token fast path that
 * the Muse Spark experiment's kernel_fn takes with moe_align_single_token (decode batches), here
 * for up to 128 slots (M * top_k <= 128) and block_m <= 16.  One launch computes exactly what
 * moe_align(topk_ids, M, top_k, expert_start, W13->n_experts, block_m, ...) followed by
 * moe_w4a16_gemm_act(..., numel = M * top_k, ...) computes, bit for bit: `out` as
 * moe_w4a16_gemm_act, and sorted_token_ids [cap], expert_ids [cap / block_m],
 * num_tokens_post_padded [1] and slot_local_ids [M * top_k] (capacity and contents as moe_align;
 * all four are outputs here, device memory owned by the caller) for the down GEMM and the
 * combine that follow.  Runs the streaming decode kernel: cfg NULL or AUTO, or kernel DECODE with
 * gemv_rows 0.  Errors: MOE_EUNSUPPORTED for more than 128 slots, block_m > 16, n_experts > 512 or
 * another kernel; otherwise as moe_align and moe_w4a16_gemm_act.
 */
int moe_w4a16_gemm_act_routed(moe_act_kind kind, float alpha, float limit, const uint16_t* A,
                              int64_t a_rows, int32_t lda, uint16_t* out, int32_t ldo,
                              const moe_weights* W13, const int32_t* topk_ids, int64_t M, int32_t top_k,
                              int32_t expert_start, int32_t block_m, int32_t* sorted_token_ids,
                              int32_t* expert_ids, int32_t* num_tokens_post_padded,
                              int32_t* slot_local_ids, const moe_gemm_config* cfg, hipStream_t stream);

/*
 * The down GEMM with the no-norm top-k weighted sum fused in (the second half of the epilogue
 * fusion the Muse Spark experiment's kernel_fn leaves to fused_post_expert_norm_weighted_sum; its
 * "no norm" branch): one launch computes what moe_w4a16_gemm(A, M * top_k, lda, y, ldy, W, ...,
 * numel = M * top_k, top_k = 1, ...) followed by moe_combine(y, topk_weights, slot_local_ids,
 * NULL, 0, routed_scaling, M, top_k, N, out) computes, bit for bit, when that GEMM runs the same
 * streaming-kernel configuration (y is still written; the summation order and roundings are the
 * combine's).  Decode batches only: block_m <= 16 and the streaming kernel: cfg kernel DECODE
 * with gemv_rows 0, or cfg NULL / AUTO for the streaming kernel's default configuration (which
 * moe_gemm_choose also returns below about 32 live slots or for K < 2048; above, it picks the
 * MFMA kernel, whose fp32 summation order differs).
 *   A, lda, y, ldy, W, sorted/expert ids, num_tokens_post_padded, block_m: as moe_w4a16_gemm
 *     (A row = slot; W a plain projection, not MOE_PREP_GATE_UP)
 *   M, top_k        tokens and slots per token (numel = M * top_k, top_k <= 64)
 *   topk_weights    device fp32 [M, top_k]; slot_local_ids device int32 [M, top_k] (moe_align's)
 *   routed_scaling  multiplies every output (1 = none)
 *   counters        device int32 [n_counters], n_counters >= M * ceil(N / (16 * ng)) (M * N / 16
 *                   suffices for every ng): arrival counts per (token, strip of output columns).
 *                   They must be zero on entry and are left zero by every completed call (clear
 *                   them once after allocation); two calls that overlap in time must not share them
 *   out             device bf16 [M, ldo], ldo >= N: every row written (zeros for tokens with no
 *                   live slot)
 * The last workgroup to store a token's rows of a column strip sums them (release fence, counter
 * increment, acquire fence), so no second launch is needed.  Errors: MOE_EUNSUPPORTED for
 * block_m > 16 or another kernel, MOE_ESIZE for too few counters, else as moe_w4a16_gemm.
 */
int moe_w4a16_gemm_combine(const uint16_t* A, int64_t a_rows, int32_t lda, uint16_t* y, int32_t ldy,
                           const moe_weights* W, const int32_t* sorted_token_ids, const int32_t* expert_ids,
                           const int32_t* num_tokens_post_padded, int64_t M, int32_t top_k, int32_t block_m,
                           const float* topk_weights, const int32_t* slot_local_ids, float routed_scaling,
                           int32_t* counters, int64_t n_counters, uint16_t* out, int32_t ldo,
                           const moe_gemm_config* cfg, hipStream_t stream);

/*
 * moe_w4a16_gemm_combine for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation and
 * result, bit for bit, with the arrival counters taken from a scratch array inside the library
 * instead of a caller workspace.  Nothing is allocated: no hipMalloc / hipFree and no allocating
 * library routine, here or in any call it makes.
 *   Arguments as moe_w4a16_gemm_combine without counters / n_counters.
 *   Limit: M * ceil(N / (16 * ng)) <= MOE_NOALLOC_MAX_COUNTERS (262144 int32, 1 MiB per device;
 *   e.g. M <= 1024 tokens for N = 4096 at ng = 2); beyond it MOE_ESIZE, nothing launched.
 * The scratch array lives in the library's device memory, one copy per GPU the library runs on,
 * held until the process ends; its device address is looked up on the first call on each
 * device (with that device current).  Each call first clears the counters it uses with a small
 * fill kernel on `stream` (no memset node, so the call may be captured in a graph), so no state
 * carries over from an earlier call.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race and give wrong results --
 * order them on one stream or use moe_w4a16_gemm_combine with separate counters.
 */
#define MOE_NOALLOC_MAX_COUNTERS 262144
int moe_w4a16_gemm_combine_noalloc(const uint16_t* A, int64_t a_rows, int32_t lda, uint16_t* y, int32_t ldy,
                                   const moe_weights* W, const int32_t* sorted_token_ids,
                                   const int32_t* expert_ids, const int32_t* num_tokens_post_padded, int64_t M,
                                   int32_t top_k, int32_t block_m, const float* topk_weights,
                                   const int32_t* slot_local_ids, float routed_scaling, uint16_t* out,
                                   int32_t ldo, const moe_gemm_config* cfg, hipStream_t stream);

/* ----------------------------------------------------------------------------- act */

/*
 * Activation over rows of the GEMM1 output (silu_and_mul of the experiment; GPT-OSS
 * swiglu_gpt_oss_sigmoid_alpha_contiguous of sglang PR 28231; the non-gated relu2):
 *   in   device bf16 [R, ld_in]: gated kinds gate = columns [0, I), up = [I, 2I) (ld_in >= 2I);
 *        MOE_ACT_RELU2 the I columns of h (ld_in >= I)
 *   out  device bf16 [R, ld_out]: I columns
 *   slot_local_ids  device int32 [R] or NULL: rows whose id is < 0 are skipped (not written)
 *   alpha, limit    SWIGLU_ALPHA only; limit = +inf disables the clamps
 * Computed in fp32 from the bf16 inputs, rounded to bf16 once.
 */
int moe_act(moe_act_kind kind, const uint16_t* in, int32_t ld_in, uint16_t* out, int32_t ld_out,
            int64_t R, int32_t I, const int32_t* slot_local_ids, float alpha, float limit,
            hipStream_t stream);

/* ----------------------------------------------------------------------------- combine */

/*
 * Top-k weighted combine, optionally after the weight-first post-expert RMSNorm
 * (_expert_norm_factors + _expert_norm_sum of the experiment):
 *   y               device bf16 [M * top_k, H]: GEMM2 output, row t*top_k+s
 *   topk_weights    device fp32 [M, top_k]
 *   slot_local_ids  device int32 [M, top_k]: slots with id < 0 are dead and contribute 0
 *                   (their y rows may be read but their values are never used)
 *   norm_w          device bf16 [H] = bf16(1 + w) (moe_norm_weight), or NULL for no norm
 *   routed_scaling_factor  multiplies every output (1 = none; the sglang PR 31552 argument)
 *   out             device bf16 [M, H], every row written (zeros for tokens with no live slot)
 * With norm: z = y * norm_w, factor = g / sqrt(sum(z^2) / H + eps), out = rsf * sum factor * z.
 * Without:   out = rsf * sum g * y.   fp32 accumulation, one bf16 rounding at the end.
 */
int moe_combine(const uint16_t* y, const float* topk_weights, const int32_t* slot_local_ids,
                const uint16_t* norm_w, float eps, float routed_scaling_factor, int64_t M,
                int32_t top_k, int32_t H, uint16_t* out, hipStream_t stream);

/* ----------------------------------------------------------------------------- fp8 requant */

/*
 * Launch hint of moe_fp8_requant (results never depend on it).
 *   workgroups  >= 1 workgroups of four waves; each wave takes every (workgroups*4)-th item
 *   unroll      work items in flight per wave: 1, 2 or 4
 */
typedef struct {
  int32_t workgroups;
  int32_t unroll;
} moe_requant_config;

/*
 * A launch hint for moe_fp8_requant on E experts of max_m row slots of K codes, a device with
 * num_cus compute units, and expected_rows live rows per expert (the dispatch's expected_m of
 * the "sglang PR 35760" summary, item 4; <= 0 = unknown: every row slot is assumed live, which
 * is what moe_fp8_requant uses when cfg is NULL).  About two 1024-byte items per wave as two,
 * four or eight workgroups per CU, never more waves than the batch can have items; a wave takes
 * two or four items at a time beyond that.  Any value is correct: only speed depends on it.  A pure host
 * function.  Errors: MOE_EINVAL for a null cfg or E, max_m < 0, K < 16, num_cus < 1.
 */
int moe_fp8_requant_choose(int32_t E, int32_t max_m, int32_t K, int32_t expected_rows,
                           int32_t num_cus, moe_requant_config* cfg);

/*
 * W4AFP8 activation requant ("sglang PR 35760" summary: "Feature and motivation",
 * "Implementation breakdown" items 1-3): float8 e4m3fn activations quantised per token and
 * group are re-expressed against one per-tensor scale.  For every live element
 *     out = e4m3fn_sat( float32( float32(x * s) * r ) ),   r = float32(1 / *tensor_scale)
 * with x the decoded code, s its (row, group) scale, and e4m3fn_sat rounding to nearest (ties
 * to the even code) after clamping the magnitude to 448, keeping the sign (-0 -> 0x80) and
 * sending NaN to 0x7F.
 *   x             device uint8 [E, max_m, K]: e4m3fn codes, row m of expert e live iff
 *                 m < clamp(masked_m[e], 0, max_m)
 *   scales        device fp32; the scale of (e, m, group g = k / group_size) is
 *                 scales[e*scale_stride_e + m*scale_stride_m + g*scale_stride_g] (elements):
 *                 row-major [E, max_m, K/group_size] is (max_m*G, G, 1); the column-major
 *                 per-expert layout [E, K/group_size, max_m] of a DeepEP dispatch is (G*max_m, 1, max_m)
 *   masked_m      device int32 [E]: live rows per expert (values outside [0, max_m] are clamped)
 *   tensor_scale  device fp32 [1]: the per-tensor scale
 *   group_size    a multiple of 16 dividing K (128 on the page)
 *   out           device uint8 [E, max_m, K]: live rows written; every other row slot is left
 *                 untouched.  out == x (in place) is allowed; any other overlap is rejected.
 *   cfg           launch hint or NULL (moe_fp8_requant_choose)
 * Nothing is read or written for row slots that are not live, so their contents are free.
 * E = 0 or max_m = 0 launches nothing.  Errors: MOE_EINVAL for null pointers, x/out not 16-byte
 * aligned, K not a positive multiple of group_size, negative strides, a bad cfg, or a partial
 * overlap; MOE_EUNSUPPORTED for group_size not a multiple of 16, more than 1024 experts or
 * E*max_m*ceil(K/1024) >= 2^31.
 */
int moe_fp8_requant(const uint8_t* x, const float* scales, int64_t scale_stride_e,
                    int64_t scale_stride_m, int64_t scale_stride_g, const int32_t* masked_m,
                    const float* tensor_scale, int32_t E, int32_t max_m, int32_t K,
                    int32_t group_size, uint8_t* out, const moe_requant_config* cfg,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_W4A16_H */
