/*
 * moe_mxfp4.h -- C ABI of a sparse Mixture-of-Experts FFN layer with MXFP4
 * routed experts and bf16 shared experts, for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (per token x, one MoE layer):
 *   Deltafin explainer (bhfrc.com), section 5.1, and Deltafin README
 *   ("An experiment in running Kimi K3 ..."), "How it works": the router picks
 *   the top-k (K3: 16) of E (K3: 896) routed experts, the selected experts'
 *   MXFP4 weights are applied with the dequantisation fused into the product
 *   (README, "Techniques / Compute"), and the outputs of the always-on shared
 *   experts (K3: 2) are added.  Readings used where the pages are silent:
 *     s_e   = sigmoid(x . Wr[e] + bias[e])        (bias optional)
 *     ids   = k largest s_e, ties to the lower expert index, ordered by
 *             (s descending, index ascending)
 *     w_j   = s_{ids_j} / sum_j s_{ids_j}
 *     E(x)  = Wd (SiLU(Wg x) * (Wu x))            SwiGLU, MXFP4 weights
 *     S(x)  = same form, bf16 weights              shared experts, weight 1
 *     y     = residual + sum_j w_j E_{ids_j}(x) + sum_s S_s(x)
 *   rounded once to bf16 (round to nearest even) at the output; everything
 *   before is accumulated in fp32.
 *
 * MXFP4 (kimi-k3-in-c note (curvesoft.net), byte accounting): 4-bit E2M1
 * elements with one E8M0 exponent per 32 consecutive elements along the
 * input dimension, 0.53125 bytes per weight, 17,547,264 bytes per K3 expert.
 *
 * Canonical expert record (README, "Techniques / I/O and streaming": an
 * expert's six tensors are one contiguous span), the interchange format:
 *     gate codes  uint8 [I][H/2]    gate scales uint8 [I][H/32]
 *     up   codes  uint8 [I][H/2]    up   scales uint8 [I][H/32]
 *     down codes  uint8 [H][I/2]    down scales uint8 [H][I/32]
 *   rows are output features, the contraction dimension is contiguous;
 *   element k of a row is in byte k/2, even k in the low nibble; scale byte j
 *   of a row covers elements 32j..32j+31 and means 2^(byte-127) (255 = NaN).
 *   moe_record_bytes() gives the size (17,547,264 at H=7168, I=1536).
 *
 * Packed layout (what the layer kernels read; moe_pack_experts writes it).
 * Each MXFP4 matrix of R rows x K columns (nb = K/32 blocks per row, nkb =
 * ceil(nb/4) code tiles per row group, nkb4 = nkb rounded up to 4) is
 *   codes:  tiles of 16 rows x 128 columns, 1 KiB each, tile (rg, kb) at
 *           byte (rg nkb + kb) 1024; its bytes 16 l .. 16 l + 15 hold the
 *           codes of block 4 kb + l/16 of row 16 rg + l%16 (zero codes past
 *           block nb);
 *   scales: after the codes; byte ((rg nkb4/4 + kb/4) 64 + l) 4 + kb%4 is
 *           that block's E8M0 exponent (127 past block nb).
 * A wave64 reads one tile as 1 KiB of contiguous codes in which lane l holds
 * exactly its MFMA operand, and the exponents of four consecutive tiles (a
 * super-step) as 256 contiguous bytes, one dword per lane.  A record is gate, up, down matrices back to back;
 * same size as the canonical record when K is a multiple of 512
 * (17,547,264 bytes at K3 shape).  bf16 shared matrices are packed into
 * 1 KiB tiles of 16 rows x 32 columns (lane l: row 16 rg + l%16, columns
 * 8 (l/16) .. +7), tile (rg, u) at element (rg K/32 + u) 512.
 *
 * Conventions for every call:
 *   - pointers are DEVICE pointers unless stated; bf16 is passed as uint16_t
 *     bit patterns; every device pointer must be 16-byte aligned.
 *   - the caller owns every buffer.  The library allocates no device memory
 *     at run time (moe_layer_scratch uses a static device array, present
 *     from load; an expert pool keeps its bookkeeping in host memory),
 *     keeps no other mutable global state (beyond two per-host-thread
 *     settings: the timing hook and the wait limit), never synchronises the
 *     host (except moe_workspace_status, a query), and enqueues all work on
 *     the given stream (NULL = the default stream).
 *   - arguments are validated on the host before anything is launched; on
 *     error nothing is launched and a negative MOE_E* code is returned.
 *     Device-side faults surface at the caller's next synchronisation.
 *   - x, y and residual must not overlap, except y == residual (in place).
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION ((3u << 16) | 0u)

/* status codes */
#define MOE_OK 0
#define MOE_EINVAL -1      /* null pointer, negative or zero size */
#define MOE_EALIGN -2      /* a device pointer or stride is not 16-byte aligned */
#define MOE_ESHAPE -3      /* unsupported shape (see moe_layer_desc) */
#define MOE_EWORKSPACE -4  /* workspace smaller than moe_workspace_bytes() */
#define MOE_EDEVICE -5     /* current device is not gfx950 */
#define MOE_ELAUNCH -6     /* a kernel launch failed; see moe_last_hip_error() */
#define MOE_EUNSUPPORTED -7 /* valid request the library does not implement */
#define MOE_ETIMEOUT -8    /* a top-k wait gave up (moe_workspace_status) */

/* moe_layer_desc.router_mode */
#define MOE_ROUTER_BIAS_LOGITS 0
#define MOE_ROUTER_BIAS_SELECT 1

/* moe_forward path selection */
#define MOE_PATH_AUTO 0  /* GEMV path for small T, MXFP8 MFMA path for large T */
#define MOE_PATH_GEMV 1  /* bf16 activations, dequant-fused GEMV (decode) */
#define MOE_PATH_MFMA 2  /* MXFP8 activations, scaled FP4 MFMA (prefill) */
#define MOE_PATH_MFMA_FP4 3  /* MXFP4 activations, scaled FP4 x FP4 MFMA (prefill; opt-in) */

/*
 * One MoE layer.  Host struct; the pointers in it are device pointers.
 *   hidden (H) and inter (I): multiples of 32, H <= 8192, I <= 8192.
 *   n_experts (E) <= 1024; 1 <= top_k <= min(E, 32); 0 <= n_shared <= 4.
 *   router_w:    bf16 [E][H]
 *   router_bias: fp32 [E], or NULL; where it enters is router_mode's choice
 *   router_mode: MOE_ROUTER_BIAS_LOGITS: the bias is added to the logits
 *                before the sigmoid, for the choice and the weights (the
 *                reading of the pages' per-expert logit bias);
 *                MOE_ROUTER_BIAS_SELECT: the bias is added to the sigmoid
 *                scores for the choice only, and the weights come from the
 *                unbiased scores (the DeepSeek-V3 report's gate, section
 *                2.1.2); other values: MOE_EINVAL
 *   routed_scale: factor on the routed combine weights (the weights
 *                moe_route returns and moe_layer applies); 0 is read as 1,
 *                so a zeroed descriptor keeps plain weights summing to 1;
 *                negative, infinite or NaN: MOE_EINVAL
 *   experts:     E PACKED records (moe_pack_experts), expert_stride bytes
 *                apart (stride >= moe_packed_record_bytes, multiple of 16).
 *                Not the canonical record: a caller holding canonical
 *                records repacks them once with moe_pack_experts (same size
 *                at K3 shape).  The packed order makes every wave-wide
 *                16-byte load one contiguous KiB that holds each lane's MFMA
 *                operand; on canonical rows the 16 lanes of a quarter-wave
 *                read 16 different rows (64 cache lines per load), which
 *                doubled the decode gate/up time when measured.
 *   shared_gate, shared_up: S packed bf16 [I][H] matrices, back to back;
 *   shared_down: S packed bf16 [H][I] matrices (moe_pack_bf16); NULL when
 *                n_shared == 0
 *   expert_slot: NULL (expert e's record is record e of `experts`), or an
 *                expert pool: device int32 [E], expert e's record is record
 *                expert_slot[e] of `experts`, which then holds n_slots
 *                records (values outside 0 .. n_slots - 1 are clamped).
 *                moe_pool_fetch (below) keeps such a pool filled from host
 *                memory; a call must only route to experts whose records
 *                are resident.  n_slots is 0 when expert_slot is NULL.
 */
typedef struct moe_layer_desc {
  int32_t hidden;
  int32_t inter;
  int32_t n_experts;
  int32_t top_k;
  int32_t n_shared;
  int32_t router_mode;
  const uint16_t* router_w;
  const float* router_bias;
  const uint8_t* experts;
  uint64_t expert_stride;
  const uint16_t* shared_gate;
  const uint16_t* shared_up;
  const uint16_t* shared_down;
  const int32_t* expert_slot;
  int32_t n_slots;
  float routed_scale;
} moe_layer_desc;

/* major << 16 | minor of the library; bindings refuse a different major. */
uint32_t moe_abi_version(void);

/* Static description of a status code (host; never NULL). */
const char* moe_status_string(int status);

/* hipError_t of the last failed launch on the calling host thread. */
int moe_last_hip_error(void);

/* Bytes of one expert record for (hidden, inter); MOE_ESHAPE if not
 * multiples of 32. */
int moe_record_bytes(int32_t hidden, int32_t inter, uint64_t* out_bytes);

/* Bytes of one packed expert record (see "Packed layout" above). */
int moe_packed_record_bytes(int32_t hidden, int32_t inter, uint64_t* out_bytes);

/*
 * Repack n_experts canonical records (src, src_stride bytes apart) into the
 * packed layout at dst (dst_stride bytes apart; dst_stride >=
 * moe_packed_record_bytes, multiple of 16).  One-time weight preparation;
 * src and dst must not overlap.  Weight loading, not part of the hot path.
 */
int moe_pack_experts(const uint8_t* src, uint64_t src_stride, uint8_t* dst, uint64_t dst_stride,
                     int32_t n_experts, int32_t hidden, int32_t inter, hipStream_t stream);

/*
 * Repack count row-major bf16 matrices of rows x cols (back to back at src)
 * into packed tiles (back to back at dst, same total size); rows a multiple
 * of 16, cols a multiple of 32.  Used for the shared experts.
 */
int moe_pack_bf16(const uint16_t* src, uint16_t* dst, int32_t count, int32_t rows, int32_t cols,
                  hipStream_t stream);

/* Workspace needed by moe_route / moe_forward / moe_layer for n_tokens
 * tokens of this layer.  The caller allocates it (any device memory, e.g. a
 * torch uint8 tensor); its contents need no initialisation and are
 * overwritten by every call (except the status marker, see
 * moe_workspace_status).  Calls that share a workspace must be ordered
 * (same stream). */
int moe_workspace_bytes(const moe_layer_desc* layer, int64_t n_tokens, uint64_t* out_bytes);

/*
 * Router: topk_ids int32 [T][k] and topk_w fp32 [T][k] (see the formulas at
 * the top).  Logits accumulate in fp32 from exact bf16 products.
 *   x: bf16 [T][H].
 */
int moe_route(const moe_layer_desc* layer, const uint16_t* x, int64_t n_tokens,
              int32_t* topk_ids, float* topk_w, void* workspace, uint64_t workspace_bytes,
              hipStream_t stream);

/*
 * Experts and combine for a given routing:
 *   y = residual + sum_j topk_w[t][j] * E_{topk_ids[t][j]}(x_t) + sum_s S_s(x_t)
 *   x, residual (or NULL), y: bf16 [T][H];  topk_ids int32 [T][k] with
 *   distinct ids per token in [0, E);  topk_w fp32 [T][k].
 *   path: MOE_PATH_GEMV keeps x and h exact (bf16 x, fp32 h);
 *         MOE_PATH_MFMA rounds x and h to MXFP8 (E4M3 with one E8M0
 *         exponent per 32 along the contraction) for the routed experts, the
 *         reading of the MXFP8 activations in the Deltafin explainer,
 *         section 2.1;
 *         MOE_PATH_MFMA_FP4 rounds them to MXFP4 instead (E2M1 with one E8M0
 *         exponent per 32 along the contraction, the weights' own format:
 *         E = clamp(floor(log2 amax) - 2), round to nearest even, saturating
 *         at 6), for the FP4 x FP4 matrix-core rate (about twice FP4 x FP8);
 *         MOE_PATH_AUTO picks MFMA when n_tokens >= moe_mfma_min_tokens()
 *         (never the FP4 variant).
 * Routing ids out of range are clamped on the device (never read out of
 * bounds); they are the caller's error.
 */
int moe_forward(const moe_layer_desc* layer, const uint16_t* x, int64_t n_tokens,
                const int32_t* topk_ids, const float* topk_w, const uint16_t* residual,
                uint16_t* y, int32_t path, void* workspace, uint64_t workspace_bytes,
                hipStream_t stream);

/*
 * moe_forward for experts that arrive while the call runs (an expert pool
 * filled on another stream; Deltafin README, I/O and streaming: the expert
 * reads overlap the compute that does not need them).  On the GEMV path the
 * shared experts (which need no routed record) are enqueued first, then
 * `stream` waits for records_ready -- an event the caller records on the
 * stream of moe_pool_fetch after the fetch -- then the routed experts and the
 * combine run.  The MFMA paths, whose shared experts share the routed
 * launches, wait before everything.  records_ready NULL: moe_forward.  The
 * caller keeps earlier work that reads the pool ordered before the fetch
 * (moe_pool_fetch overwrites slots on its own stream).
 */
int moe_forward_pooled(const moe_layer_desc* layer, const uint16_t* x, int64_t n_tokens,
                       const int32_t* topk_ids, const float* topk_w, const uint16_t* residual,
                       uint16_t* y, int32_t path, void* workspace, uint64_t workspace_bytes,
                       hipEvent_t records_ready, hipStream_t stream);

/* moe_route followed by moe_forward, scheduled together (the shared experts
 * overlap the router).  topk_ids / topk_w receive the routing. */
int moe_layer(const moe_layer_desc* layer, const uint16_t* x, int64_t n_tokens,
              const uint16_t* residual, uint16_t* y, int32_t* topk_ids, float* topk_w,
              int32_t path, void* workspace, uint64_t workspace_bytes, hipStream_t stream);

/*
 * Status of the calls that used a workspace.  For up to 8 tokens on the GEMV
 * path, moe_layer runs the top-k inside the router launch, in a workgroup
 * that waits for the other workgroups' logits; for one token the whole
 * layer is that launch, whose routed and shared workgroups also wait for
 * the top-k's expert ids and for the gate/up results they consume.  Every
 * such wait is bounded (see moe_set_wait_limit).  If one ever gives up, the
 * call's routing (and output) is wrong, and the first 8 bytes of its
 * workspace are set to a marker that no call clears.  moe_workspace_status
 * synchronises `stream` (the stream of those calls), reads the marker and
 * returns MOE_ETIMEOUT if it is set -- clearing it, so a later query reports
 * only later calls -- else MOE_OK.  A workspace whose first bytes were never
 * written by a call reads as MOE_OK.  Host-synchronous (unlike every other
 * call).
 */
int moe_workspace_status(const void* workspace, uint64_t workspace_bytes, hipStream_t stream);

/*
 * Polls (~0.3 us each) after which the top-k wait above gives up, for calls
 * made later from the calling host thread; negative restores the default
 * (2^20, ~0.3 s).  A diagnostic and test knob: 0 makes every such wait give
 * up at once, so the failure path can be exercised with every kernel still
 * exiting normally.
 */
int moe_set_wait_limit(int64_t polls);

/*
 * Test export: where a region of the workspace of a call with n_tokens
 * tokens lives (*offset bytes from its start, *bytes long), so that tests
 * can compare the layer's intermediate values with an independent model.
 * Kq = H and Iq = I rounded up to multiples of 512.  Scale rows are in
 * "MFMA order": the byte of block b of a row is at position
 * (b & ~15) | ((b & 3) << 2) | ((b & 15) >> 2).
 *   MOE_WS_PAIRS:    int32 [T k]: the pair t k + j at each plan position
 *                    (pairs grouped by expert, experts ascending); written
 *                    by every call except single-token GEMV calls
 *   MOE_WS_X_CODES:  uint8 E4M3 [T][Kq] MXFP8 codes of x (MFMA path; zero
 *                    codes past H); on the MXFP4 path the first T Kq / 2
 *                    bytes hold [T][Kq / 2] E2M1 codes, two per byte, even
 *                    element in the low nibble
 *   MOE_WS_X_SCALES: uint8 E8M0 [T][Kq/32], MFMA order (127 past H)
 *   MOE_WS_H_CODES:  uint8 E4M3 [T k][Iq]: MXFP8 codes of SiLU(g) u of the
 *                    pair at each plan position (MFMA path); MXFP4 path:
 *                    [T k][Iq / 2] E2M1 codes in the first T k Iq / 2 bytes
 *   MOE_WS_H_SCALES: uint8 E8M0 [T k][Iq/32], MFMA order
 * Contents are those of the last call on the workspace once its stream has
 * reached that point.
 */
#define MOE_WS_PAIRS 0
#define MOE_WS_X_CODES 1
#define MOE_WS_X_SCALES 2
#define MOE_WS_H_CODES 3
#define MOE_WS_H_SCALES 4
int moe_workspace_region(const moe_layer_desc* layer, int64_t n_tokens, int32_t region,
                         uint64_t* offset, uint64_t* bytes);

/*
 * moe_layer for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same call
 * without a workspace argument.  Its workspace is a static device array of
 * MOE_SCRATCH_BYTES that the library holds on each device it runs on until
 * the process ends; the call allocates nothing and calls no allocating
 * routine.  A call whose workspace (moe_workspace_bytes) exceeds
 * MOE_SCRATCH_BYTES returns MOE_EWORKSPACE and launches nothing (at the K3
 * shape: up to 64 tokens fit).  Every call on a device shares that device's
 * array: calls that overlap on one device (other streams, other host
 * threads) race and must be ordered by the caller.  The array keeps the last
 * call's contents; nothing in it needs clearing between calls.  A top-k wait
 * that gives up (see moe_workspace_status) cannot be queried for these calls.
 */
#define MOE_SCRATCH_BYTES (64ull << 20)
int moe_layer_scratch(const moe_layer_desc* layer, const uint16_t* x, int64_t n_tokens,
                      const uint16_t* residual, uint16_t* y, int32_t* topk_ids, float* topk_w,
                      int32_t path, hipStream_t stream);

/* Smallest n_tokens for which MOE_PATH_AUTO takes the MFMA path. */
int64_t moe_mfma_min_tokens(void);

/*
 * RMSNorm for stacked layers: out = bf16(x * (mean(x^2) + eps)^-1/2 * gamma),
 * fp32 inside.  x, out: bf16 [T][H] (may be equal); gamma: bf16 [H].
 */
int moe_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int64_t n_tokens,
                int32_t hidden, uint16_t* out, hipStream_t stream);

/*
 * Expert pool: the experts are not all resident in HBM.
 *
 * Deltafin README, I/O and streaming, and the Deltafin explainer, section
 * 6.1: the model does not fit the machine, so each token's selected experts
 * are read from storage into memory as whole contiguous records (17.5 MB at
 * the K3 shape), and records the previous tokens used are kept.  Here the
 * records live in host memory (pinned, so the copies are DMA), and a pool of
 * n_slots records in HBM holds the resident ones; a layer descriptor with
 * expert_slot = the pool's slot map and experts = the pool runs on them.
 *
 * moe_pool_create: host_records (host, pinned for asynchronous copies): E
 *   PACKED records, stride bytes apart; slots (device): n_slots records,
 *   stride bytes apart; slot_map (device int32 [E]): written by the pool,
 *   every entry 0 until its expert is fetched.  1 <= n_slots <= E; stride a
 *   multiple of 16.  The caller owns all three buffers and keeps them alive
 *   until moe_pool_destroy; the pool holds host-side bookkeeping only.
 *   Enqueues the slot map's initialisation on stream.
 * moe_pool_fetch: makes the n_ids experts in ids (host int32, repeats
 *   allowed, each in 0 .. E-1) resident: a record not in the pool is copied
 *   host -> device on stream into a free slot, else into the slot used
 *   longest ago by an expert not in ids, and the slot map is updated on
 *   stream.  More distinct experts than n_slots: MOE_ESHAPE, nothing done.
 *   *copied (may be NULL) receives the number of records copied.  Work is
 *   ordered on stream, so kernels enqueued before it that read the pool
 *   finish before a slot is overwritten, and layer calls enqueued after it
 *   see the records.  Calls on one pool must not run concurrently.  A
 *   failed copy or launch returns MOE_ELAUNCH and empties the pool's
 *   bookkeeping (no record counts as resident until fetched again).
 * moe_pool_stats: records fetched so far (copied) and found resident.
 */
typedef struct moe_expert_pool moe_expert_pool;
int moe_pool_create(const uint8_t* host_records, uint64_t stride, int32_t n_experts,
                    uint8_t* slots, int32_t n_slots, int32_t* slot_map, hipStream_t stream,
                    moe_expert_pool** out_pool);
int moe_pool_fetch(moe_expert_pool* pool, const int32_t* ids, int64_t n_ids, hipStream_t stream,
                   int32_t* copied);
int moe_pool_stats(const moe_expert_pool* pool, int64_t* copied, int64_t* resident);
int moe_pool_destroy(moe_expert_pool* pool);

/*
 * Optional per-kernel timing for benchmarks.  While an event array is set
 * (per host thread), every call that launches layer kernels (moe_route,
 * moe_forward, moe_layer) or the int8 expansion has its i-th kernel stamp
 * events[2i] with its start and events[2i+1] with its end, while
 * 2i + 1 < n_events: the dispatch takes the timestamps
 * (hipExtLaunchKernelGGL), so a pair spans exactly that kernel's execution,
 * as a kernel trace measures it.  moe_profile_count() returns how many
 * events the last call into the library stamped (twice its timed kernels;
 * 0 after calls that launch none of these).  Kernel order:
 * moe_route: router logits, top-k;
 * moe_forward (GEMV path): plan + shared gate/up, shared down + routed
 * gate/up, routed down + combine; moe_layer (GEMV path): router logits +
 * shared gate/up, top-k + plan + shared down, routed gate/up, routed down
 * + combine -- for 2 to 8 tokens: router logits + shared gate/up + top-k
 * and plan, shared down + routed gate/up, routed down + combine; for one
 * token: the whole layer (router logits, shared gate/up, top-k, routed
 * gate/up and down, shared down, combine) in one launch;
 * moe_layer (MFMA path): x to MXFP8 + router logits, top-k + plan, routed +
 * shared gate/up, routed + shared down, combine; moe_forward (MFMA path):
 * plan + x to MXFP8, then the same last three.  The caller creates and owns the hipEvent_t
 * handles; pass NULL / 0 to stop.  Timing only attaches events to the
 * launches; no kernel is skipped or changed.
 */
int moe_profile_events(hipEvent_t* events, int32_t n_events);
int moe_profile_count(void);

/*
 * Test export: the fp32 weights of one matrix of one (packed) expert,
 * decoded by the same device conversion the expert kernels use and written
 * in canonical order.  expert: the record's index in layer->experts (for
 * a pool, its slot: 0 .. n_slots-1).  matrix: 0 gate [I][H], 1 up [I][H],
 * 2 down [H][I]; out: fp32 of that shape.
 */
int moe_dequant_export(const moe_layer_desc* layer, int32_t expert, int32_t matrix, float* out,
                       hipStream_t stream);

/*
 * Test export: MXFP8 quantisation of bf16 rows as used by the MFMA path.
 *   x: bf16 [T][K] (K multiple of 32); codes: uint8 [T][K] E4M3;
 *   scales: uint8 [T][K/32] E8M0.
 */
int moe_mxfp8_quantize(const uint16_t* x, int64_t n_rows, int32_t k, uint8_t* codes,
                       uint8_t* scales, hipStream_t stream);

/*
 * Row-scaled int8 -> fp32 expansion of a dense weight matrix (Deltafin
 * README, Techniques / Compute: the non-expert weights are kept as int8
 * with one scale per row, and a fused kernel converts, scales and copies
 * them into the fp32 weights, bit-exact against the unfused path).
 *   q:     device int8 [rows][cols], row-major, 4-byte aligned
 *   scale: device fp32 [rows], 4-byte aligned
 *   out:   device fp32 [rows][cols], 16-byte aligned; must not overlap q
 *   out[r][c] = (float)q[r][c] * scale[r], one fp32 rounding (IEEE: a zero
 *   times a negative scale is -0, times inf or NaN is NaN).
 *   cols a multiple of 4 and rows * cols <= 2^40, else MOE_ESHAPE.  One
 *   launch on stream; nothing allocated.
 */
int moe_int8_row_dequant(const int8_t* q, const float* scale, int64_t rows, int64_t cols,
                         float* out, hipStream_t stream);

/*
 * Measurement export: the issue rate of the block-scaled 16x16x128 MFMA for
 * an operand-format pair, the fact the choice between MXFP8 and MXFP4
 * activations for the prefill matrix cores turns on (Deltafin explainer,
 * section 2.1: MXFP4 weights with MXFP8 activations).  Formats: 4 = FP4
 * E2M1, 0 = FP8 E4M3; supported pairs (a, b) = (4, 4), (4, 0), (0, 0), else
 * MOE_EUNSUPPORTED.  Launches n_blocks workgroups of 4 waves; each wave
 * issues iters x 8 MFMAs (2 x 16 x 16 x 128 FLOP each) on register
 * operands with eight independent accumulators, and writes one checksum
 * float to out[n_blocks * 4] (device, 4-byte aligned).  Time the launch with
 * moe_profile_events.
 */
int moe_mfma_rate(int32_t a_fmt, int32_t b_fmt, int64_t iters, int32_t n_blocks, float* out,
                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
