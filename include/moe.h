/*
 * moe.h -- C ABI of the routed Mixture-of-Experts FFN layer on block-quantized experts,
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer is the GPU work under the expert-offloading systems described in
 *   [T]  "tinyserve -- MoE Expert Offloading for Consumer GPUs" (README), and
 *   [L]  llama.cpp discussion "Experiment: fixed GPU expert working set with Native CPU
 *        miss execution for Qwen sparse MoE".
 * It has five stages, each one entry point below, plus one fused call:
 *   moe_route       router GEMV, top-k, softmax over the chosen k     ([L] original post:
 *                   the router stays on the GPU; [T] "Performance": top_k = 4)
 *   moe_bucket      group the (token, choice) pairs by expert          ([T] "How it works" 6)
 *   moe_expert_ffn  gate / up / SwiGLU / down on the experts' native block-quantized bytes,
 *                   reached through an expert -> slot map into a resident pool
 *                   ([T] "How it works" 2 and 3; [L] original post: fixed packed GPU pool;
 *                   [L] "Formal gate results": mapping rewrite -> grouped quantized matmul)
 *   moe_combine     weighted merge of the k expert outputs per token  ([L] original post)
 *   moe_layer       all of the above on one stream
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers owned by the caller, 16-byte aligned unless
 *     said otherwise. The library never allocates, frees or synchronises: every call only
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the default stream) and returns.
 *     The fused call issues no host<->device traffic, so it can be captured in a HIP graph.
 *   - bf16 values are passed as uint16_t bit patterns. Logits, gate weights, the expert
 *     outputs y and the layer output are fp32. The hidden activation h (after SwiGLU) is the
 *     one bf16 rounding point inside the layer (round to nearest even).
 *   - Argument errors are detected on the host before anything is enqueued and return
 *     MOE_ERR_INVALID_ARG; moe_last_error() then holds a description (thread-local).
 *     A failed launch returns MOE_ERR_HIP with the HIP error text.
 *   - Limits: 1 <= k <= 8, k <= E <= 256, H and I multiples of 32, T >= 0. T = 0 enqueues
 *     nothing and returns MOE_OK, except moe_bucket, which then writes all-zero counts and
 *     offsets.
 *
 * Notation: T tokens, H hidden size, I expert intermediate size, E experts, k choices per
 * token, S pool slots. A pair is p = t*k + j, the j-th choice of token t.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_HIP = 3
} moe_status;

/* Block formats of the expert weights ([T] "How it works" 2 and "Formats": MXFP4 and the
 * GGUF formats computed natively).
 * MOE_W_MXFP4: blocks of 32 E2M1 codes (4 bits each) sharing one E8M0 scale byte;
 *              weight = E2M1(code) * 2^(scale - 127). Scale bytes 1..254 are supported.
 * MOE_W_Q8_0:  blocks of 32 int8 codes sharing one fp16 scale d; weight = d * q.
 * MOE_W_Q4_K:  k-quant super-blocks of 256 elements = 8 blocks of 32; block b has a 6-bit
 *              scale sc_b and a 6-bit min m_b, the super-block fp16 d and dmin;
 *              weight = d * sc_b * q - dmin * m_b for the 4-bit code q (0..15). The
 *              reduction dimension (H for gate/up, I for down) must be a multiple of 256.
 * MOE_W_Q5_K:  Q4_K's scales and mins with a 5-bit code q = low nibble + 16 * high bit
 *              (0..31); the same multiple-of-256 rule.
 * MOE_W_Q6_K:  k-quant super-blocks of 256 elements = 16 sub-blocks of 16 with a signed
 *              8-bit scale sc_j each and an fp16 d per super-block; weight = d * sc_j *
 *              (q - 32) for the 6-bit code q = low nibble + 16 * high part (0..63); the
 *              same multiple-of-256 rule.                                               */
typedef enum {
  MOE_W_MXFP4 = 1, MOE_W_Q8_0 = 2, MOE_W_Q4_K = 3, MOE_W_Q5_K = 4, MOE_W_Q6_K = 5
} moe_wfmt;

/* Which expert-FFN schedule to use. AUTO picks the GEMV schedule for T <= 16 and the
 * grouped MFMA GEMM otherwise. Both give results within the same tolerance; they are not
 * bitwise equal to each other.
 * PERSISTENT (moe_layer only; the stage calls treat it as GEMV): for 1 <= T <= 4 tokens,
 * T * E <= 256 and H <= 4096, the layer after the router's partial logits is one
 * persistent kernel -- routing, gate/up + SwiGLU, down and combine -- whose workgroups
 * hand each expert's h over through device-scope counters ([L] original post: launch
 * overhead matters at decode; [T] "How it works" 2: gate, up and down launches per
 * expert). It meets the same tolerances; on the workloads measured here it is no faster
 * than the default launch sequence, so AUTO does not choose it. Other shapes run GEMV. */
typedef enum {
  MOE_PATH_AUTO = 0, MOE_PATH_GEMV = 1, MOE_PATH_GROUPED = 2, MOE_PATH_PERSISTENT = 3
} moe_path;

/*
 * Resident expert pool ([T] "How it works" 3: a GPU slot map in front of cached experts;
 * [L] original post: a fixed subset of packed experts materialised in a GPU pool).
 *
 * Three matrices per slot: gate [I x H], up [I x H], down [H x I] (rows x K, the
 * reduction dimension K is contiguous within a block). Each matrix has a code plane and a
 * scale plane, stored in the library's TILED layout (produced by moe_pool_pack):
 *   nb = K / 32 blocks per row; a row group is 16 consecutive rows;
 *   unit(r, b) = ((r / 16) * nb + b) * 16 + (r % 16)
 *   MXFP4 codes : 16 bytes at unit(r,b) * 16; byte j holds element 2j of the block in its
 *                 low nibble and element 2j+1 in its high nibble
 *   MXFP4 scales: 1 byte at unit(r,b)
 *   Q8_0  codes : 32 bytes at unit(r,b) * 32, element i of the block at byte i
 *   Q8_0  scales: fp16 at byte unit(r,b) * 2
 *   Q4_K  codes : 16 bytes per unit; in each dword (8 consecutive elements of the block)
 *                 byte j holds element j in its low nibble and element j+4 in its high
 *                 nibble (so that each nibble plane widens to element pairs directly)
 *   Q4_K  scales: sc_b | m_b << 8 (two bytes) at byte unit(r,b) * 2; then, from byte
 *                 rows * nb * 2 of the matrix's scale plane, d | dmin << 16 (fp16 bits, four
 *                 bytes) of row r's super-block s at ((r / 16) * nsb + s) * 16 + r % 16
 *                 (nsb = K / 256), times 4
 *   Q5_K  codes : the low nibbles as Q4_K's codes; then, from byte rows * nb * 16 of the
 *                 matrix's code plane, one dword per unit at unit(r,b) * 4 whose bit 8j + s
 *                 is the high bit of element 8 (s / 2) + j + 4 (s % 2) of the block
 *   Q5_K  scales: as Q4_K
 *   Q6_K  codes : the low nibbles as Q4_K's codes; then, from byte rows * nb * 16, two
 *                 dwords per unit at unit(r,b) * 8: dword g covers code dwords 2g, 2g+1 of
 *                 the unit, its bits 8j + s and 8j + s + 1 (s = 0, 2, 4, 6) holding the
 *                 2-bit high part of element 8 (2g + s / 4) + j + 4 ((s / 2) % 2)
 *   Q6_K  scales: the two sub-block scales (int8) of block b at unit(r,b) * 2; then, from
 *                 byte rows * nb * 2, d (fp16 bits, in a four-byte record whose high half
 *                 is unused) tiled as Q4_K's (d, dmin)
 * so the 16 rows of a row group are interleaved block by block: one 64-lane 16-byte load
 * reads 16 rows x 4 MXFP4 blocks (or 16 rows x 2 Q8_0 blocks) from one contiguous KiB.
 * Slot s of a plane starts at s * (bytes per matrix); rows of a matrix must be a multiple
 * of 16 (always true, since H and I are multiples of 32).
 */
typedef struct {
  int32_t fmt;      /* moe_wfmt */
  int32_t n_slots;  /* S >= 1 */
  int32_t H, I;
  const void* gate_q; const void* gate_s;
  const void* up_q;   const void* up_s;
  const void* down_q; const void* down_s;
} moe_pool;

/* Bytes of one matrix's code plane (scales = 0) or scale plane (scales != 0) for one slot
 * of the tiled pool; 0 for an unknown format, or for a k-quant with K not a multiple of 256.
 * (The canonical planes moe_pool_pack reads are the same size, except Q6_K's canonical
 * scale plane: K/16 + K/128 bytes per row against the pool's K/16 + K/64.) */
size_t moe_plane_bytes(int32_t fmt, int32_t rows, int32_t K, int32_t scales);

/*
 * moe_pool_pack -- convert n_mats matrices [rows x K] from the CANONICAL layout into the
 * tiled pool layout above (device to device, on `stream`). This is the "mapping" step
 * a loader runs when an expert lands in a slot; it is not on the per-token path.
 * Canonical layout (row-major, per matrix):
 *   MXFP4: codes u8 [rows][K/2] (element 2j in the low nibble of byte j),
 *          scales u8 [rows][K/32]
 *   Q8_0 : codes i8 [rows][K], scales fp16 [rows][K/32]
 *   Q4_K : codes u8 [rows][K/2] (as MXFP4), scales u8 [rows][K/16 + K/64]: per row the
 *          pairs (sc_b, m_b) of its K/32 blocks, then the fp16 pairs (d_s, dmin_s) of its
 *          K/256 super-blocks (little-endian)
 *   Q5_K : codes u8 [rows][K/2 + K/8]: per row the low nibbles (as Q4_K), then the high
 *          bits (element 8j + i in bit i of byte j); scales as Q4_K
 *   Q6_K : codes u8 [rows][K/2 + K/4]: per row the low nibbles (as Q4_K), then the 2-bit
 *          high parts (element 4j + i in bits 2i, 2i+1 of byte j); scales u8
 *          [rows][K/16 + K/128]: per row the int8 sub-block scales, then fp16 d per
 *          super-block
 * src and dst must not overlap. Returns MOE_ERR_INVALID_ARG for rows % 16 != 0 or
 * K % 32 != 0 (K % 256 != 0 for the k-quants), MOE_ERR_UNSUPPORTED for an unknown fmt.
 */
moe_status moe_pool_pack(int32_t fmt, int32_t n_mats, int32_t rows, int32_t K,
                         const void* src_q, const void* src_s, void* dst_q, void* dst_s,
                         void* stream);

/*
 * moe_route -- router GEMV + top-k + softmax over the chosen k.
 *   x        bf16 [T][H] activations
 *   w_router bf16 [E][H] router weights
 *   bias     fp32 [E] added to every token's logits, or NULL
 *   topk_ids int32 [T][k] (out): for each token the k largest logits
 *            L[t,e] = sum_h x[t,h] * w_router[e,h] + bias[e], in descending order; equal
 *            logits go to the lower expert index
 *   topk_w   fp32 [T][k] (out): w[t,j] = exp(L_j - L_0) / sum_{i<k} exp(L_i - L_0)
 *   scratch  device memory of at least moe_route_scratch_bytes(T, H, E) bytes, or NULL
 *            when that function returns 0. Logits are accumulated in fp32 from exact
 *            bf16 products.
 */
size_t moe_route_scratch_bytes(int32_t T, int32_t H, int32_t E);
moe_status moe_route(const uint16_t* x, const uint16_t* w_router, const float* bias,
                     int32_t T, int32_t H, int32_t E, int32_t k,
                     int32_t* topk_ids, float* topk_w,
                     void* scratch, size_t scratch_bytes, void* stream);

/*
 * moe_bucket -- stable counting sort of the T*k pairs by expert ([T] "How it works" 6:
 * tokens grouped by expert so each expert is loaded once).
 *   topk_ids int32 [T*k], every value in [0, E) (values outside are a caller error and
 *            give unspecified buckets, never an out-of-bounds access)
 *   counts   int32 [E]   (out) pairs per expert
 *   offsets  int32 [E+1] (out) exclusive prefix sum of counts; offsets[E] = T*k
 *   perm     int32 [T*k] (out) perm[pos] = p, pairs of one expert in ascending p
 *   inv_perm int32 [T*k] (out) inv_perm[p] = pos
 *   scratch  at least moe_bucket_scratch_bytes(T, k, E) bytes (may be NULL if that is 0)
 * Bit-exact and deterministic: no ordering decision depends on atomics.
 */
size_t moe_bucket_scratch_bytes(int32_t T, int32_t k, int32_t E);
moe_status moe_bucket(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                      int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                      void* scratch, size_t scratch_bytes, void* stream);

/*
 * moe_expert_ffn -- for every bucket position pos of expert e (offsets[e] <= pos <
 * offsets[e+1]), with token t = perm[pos] / k and slot s = slot_map[e]:
 *   g = W_gate[s] x[t],  u = W_up[s] x[t]              (fp32 accumulation)
 *   h[pos] = bf16_RNE(silu(g) * u),  silu(z) = z / (1 + exp(-z))
 *   y[pos] = W_down[s] h[pos]                          (fp32)
 *   x  bf16 [T][H];  h bf16 [T*k][I] (out);  y fp32 [T*k][H] (out)
 *   offsets/perm as produced by moe_bucket for the same T, k, E.
 *   slot_map[e] == MOE_SLOT_MISS marks a non-resident expert: its h and y rows are written
 *   as zeros and no flag is raised (see moe_miss_list / moe_merge_misses).
 *   err_flags uint32 (nullable): if slot_map[e] is any other value outside [0, n_slots),
 *   that expert's h and y rows are written as zeros and bit 0 of *err_flags is set
 *   (atomic OR); nothing traps.
 *   path: moe_path.
 */
moe_status moe_expert_ffn(const moe_pool* pool, const int32_t* slot_map, int32_t E,
                          const uint16_t* x, int32_t T, int32_t k,
                          const int32_t* offsets, const int32_t* perm,
                          uint16_t* h, float* y, uint32_t* err_flags, int32_t path,
                          void* stream);

/*
 * The two halves of moe_expert_ffn, for callers that schedule them separately (the pages'
 * per-expert forward is "gate, up, down"; here gate and up share one pass):
 *   moe_expert_gate_up  writes h only (same arguments and meaning as moe_expert_ffn)
 *   moe_expert_down     y[pos] = W_down[slot_map[e]] h[pos] for every bucket position
 * Calling gate_up then down with the same path equals moe_expert_ffn.
 */
moe_status moe_expert_gate_up(const moe_pool* pool, const int32_t* slot_map, int32_t E,
                              const uint16_t* x, int32_t T, int32_t k,
                              const int32_t* offsets, const int32_t* perm, uint16_t* h,
                              uint32_t* err_flags, int32_t path, void* stream);
moe_status moe_expert_down(const moe_pool* pool, const int32_t* slot_map, int32_t E,
                           int32_t T, int32_t k, const int32_t* offsets, const uint16_t* h,
                           float* y, uint32_t* err_flags, int32_t path, void* stream);

/*
 * moe_combine -- out[t,:] = sum_{j<k} topk_w[t,j] * y[inv_perm[t*k+j], :], summed in
 * increasing j, fp32. y fp32 [T*k][H], out fp32 [T][H].
 */
moe_status moe_combine(const float* y, const int32_t* inv_perm, const float* topk_w,
                       int32_t T, int32_t k, int32_t H, float* out, void* stream);

/*
 * Resident hits and misses ([L] original post: the selected experts are split into
 * resident hits, served from the GPU pool, and misses computed elsewhere; the weighted
 * outputs are then merged; the same post proposes hit/miss counters).
 *
 * A slot_map entry MOE_SLOT_MISS marks an expert that is not in the pool. The expert FFN
 * writes zeros for its pairs and the combine therefore sums the resident pairs only.
 *
 * moe_miss_list -- the pairs routed to non-resident experts.
 *   slot_map int32 [E]; offsets int32 [E+1], perm int32 [T*k] as from moe_bucket
 *   miss_pos     int32 [T*k] (out): the missed pairs' bucket positions, increasing, in
 *                its first n_miss entries (the rest is left untouched)
 *   miss_of_pair int32 [T*k] (out): for pair p = t*k + j, its index into miss_pos, or -1
 *   counters     int32 [4] (out): resident pairs, missed pairs (n_miss), resident experts
 *                with pairs, non-resident experts with pairs
 *   A caller gathers x rows perm[miss_pos[i]] / k, computes those pairs' expert outputs
 *   y_miss[i] elsewhere, and adds them with moe_merge_misses.
 *
 * moe_merge_misses -- out[t,:] += topk_w[t,j] * y_miss[miss_of_pair[t*k+j], :] for every
 *   missed pair of token t, in increasing j (fp32, fused multiply-add).
 *   out fp32 [T][H] (in/out); y_miss fp32 [n_miss][H]; miss_of_pair and topk_w as above.
 */
#define MOE_SLOT_MISS (-1)
moe_status moe_miss_list(const int32_t* slot_map, int32_t E, const int32_t* offsets,
                         const int32_t* perm, int32_t T, int32_t k, int32_t* miss_pos,
                         int32_t* miss_of_pair, int32_t* counters, void* stream);
moe_status moe_merge_misses(float* out, const float* y_miss, const int32_t* miss_of_pair,
                            const float* topk_w, int32_t T, int32_t k, int32_t H,
                            void* stream);

/*
 * Workspace of the fused call: byte offsets (from the workspace base) of every
 * intermediate, so a caller can read them back. All offsets are 256-byte aligned.
 */
/*
 * Staged prefill ([L] "Formal gate results": for a large prefill batch the unique experts
 * picked by the router are copied in bulk into shared GPU staging windows, the mapping is
 * rewritten to those slots and the grouped quantized matmul runs on the rewritten map;
 * [T] "How it works" 6: each expert of a batch is loaded once).
 *
 * moe_stage_plan -- the mapping rewrite.
 *   counts       int32 [E]: pairs per expert (moe_bucket's counts)
 *   slot_map     int32 [E]: resident slot, or MOE_SLOT_MISS
 *   first_slot, n_stage: the window is pool slots [first_slot, first_slot + n_stage)
 *   slot_map_out int32 [E] (out; may be slot_map itself): the experts with pairs and no
 *                slot take the window's slots in increasing expert index,
 *                slot_map_out[e] = first_slot + i for the i-th of them while i < n_stage;
 *                every other entry is copied (experts beyond the window stay
 *                MOE_SLOT_MISS and take the miss path above)
 *   copy_list    int32 [E] (out): copy_list[i] = the expert staged into slot first_slot + i,
 *                for i < counters[0]; later entries are left untouched
 *   counters     int32 [2] (out): experts staged, experts left out because the window is
 *                full
 *
 * moe_stage_copy -- the bulk copy into the window.
 *   pool     the pool whose window slots are written (its planes are written through the
 *            const pointers, for slots first_slot + i, i < min(counters[0], max_copies))
 *   backing  a pool of the same format and shape in which slot e holds expert e (any
 *            memory the device can read)
 *   copy_list, counters: from moe_stage_plan (read on the device, so no host round trip
 *            is needed between the plan and the copy)
 *   max_copies: the window size n_stage given to the plan; the launch is sized for it
 *   err_flags uint32 (nullable): bit 0 is set if a listed expert is outside the backing
 *            store; that copy is skipped.
 *   Errors: MOE_ERR_INVALID_ARG if the window does not fit in the pool, or the backing
 *   store differs from the pool in format or shape.
 */
moe_status moe_stage_plan(const int32_t* counts, const int32_t* slot_map, int32_t E,
                          int32_t first_slot, int32_t n_stage, int32_t* slot_map_out,
                          int32_t* copy_list, int32_t* counters, void* stream);
moe_status moe_stage_copy(const moe_pool* pool, const moe_pool* backing,
                          const int32_t* copy_list, const int32_t* counters, int32_t first_slot,
                          int32_t max_copies, uint32_t* err_flags, void* stream);

typedef struct {
  size_t total;
  size_t topk_ids, topk_w, counts, offsets, perm, inv_perm, h, y, scratch;
  size_t act;       /* int32 list of the active experts, written for small batches */
  size_t sync;      /* int32 words the decode kernels synchronise through (H/16 + 256) */
} moe_ws_layout;

moe_status moe_layer_workspace(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                               moe_ws_layout* out);

/*
 * moe_layer -- route, bucket, expert FFN and combine for T tokens, enqueued on one stream.
 * out fp32 [T][H]. workspace: at least moe_layer_workspace(...).total bytes, 256-byte
 * aligned; its contents on entry do not matter. Calls that share a workspace must not
 * overlap in time. Small batches take shorter launch sequences: for T <= 16 and E <= 128
 * one single-workgroup kernel routes, takes the top-k, bucket-sorts the pairs and lists
 * the active experts; on the GEMV path with T*k <= 8 one kernel does the down projection
 * and the combine (each workgroup owns 16 output columns across all active experts, so no
 * atomics are involved). Results equal calling the stage entry points in order with the
 * same path.
 */
moe_status moe_layer(const moe_pool* pool, const int32_t* slot_map,
                     const uint16_t* w_router, const float* bias, const uint16_t* x,
                     int32_t T, int32_t E, int32_t k, float* out,
                     void* workspace, size_t workspace_bytes, uint32_t* err_flags,
                     int32_t path, void* stream);

/*
 * moe_layer_timed -- moe_layer, plus hipEventRecord of two caller-owned events (hipEvent_t,
 * NULL to skip) on `stream` immediately before and after the gate/up launch, so a caller
 * can time the layer's dominant kernel without a profiler. While `stream` is being captured
 * into a HIP graph the records are made with hipEventRecordExternal, so they become event
 * nodes of the graph and every replay re-records them. Same results as moe_layer.
 */
moe_status moe_layer_timed(const moe_pool* pool, const int32_t* slot_map,
                           const uint16_t* w_router, const float* bias, const uint16_t* x,
                           int32_t T, int32_t E, int32_t k, float* out,
                           void* workspace, size_t workspace_bytes, uint32_t* err_flags,
                           int32_t path, void* stream, void* ev_gate_up_begin,
                           void* ev_gate_up_end);

/*
 * moe_layer_noalloc -- moe_layer for callers that cannot allocate device memory: code that
 * runs under HIP graph capture and may not call hipMalloc, tight serving loops, and
 * harnesses that forbid allocation. Same arguments and results as moe_layer, without the
 * workspace: the layer's intermediates live in a static device array of
 * MOE_NOALLOC_WS_BYTES bytes that the library holds on each device it runs on until the
 * process ends. The call enqueues the same kernels and allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).
 *   Limit: the layer's workspace (moe_layer_workspace(...).total) must fit in
 *   MOE_NOALLOC_WS_BYTES; larger calls return MOE_ERR_INVALID_ARG and launch nothing.
 *   The first call on a device looks up the array's device address (hipGetSymbolAddress,
 *   with the stream's device current); make that first call outside a stream capture.
 *   Every call on a device shares that device's array and leaves its contents there: calls
 *   that overlap in time on one device race, as calls sharing a moe_layer workspace do.
 */
#define MOE_NOALLOC_WS_BYTES (32u << 20)
moe_status moe_layer_noalloc(const moe_pool* pool, const int32_t* slot_map,
                             const uint16_t* w_router, const float* bias, const uint16_t* x,
                             int32_t T, int32_t E, int32_t k, float* out, uint32_t* err_flags,
                             int32_t path, void* stream);

const char* moe_status_string(moe_status s);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
