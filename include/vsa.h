/*
 * vsa.h - C ABI of the MI355X (gfx950) block-sparse attention library.
 *
 * The library computes softmax attention restricted to a boolean map over
 * (Q block, KV block) pairs, forward and backward, as described on these pages:
 *   [FV-test]  FastVideo fastvideo-kernel/tests/test_vsa256_backward.py
 *              (VSA-256 parity tests: 256-token tiles, per-tile valid counts,
 *              top-k tile selection, the gated compression branch, BHSD/BSHD,
 *              inference vs training forward, LSE shape [B,H,S]);
 *   [FV-cute]  FastVideo fastvideo_kernel/block_sparse_attn_cute_fwd.py
 *              (`_map_to_index`: block map -> per-row block lists;
 *              `_build_vbs_mask_mod`: per-tile valid-token predicate;
 *              `_build_sparse_tensors`: Q-owned forward index, KV-owned
 *              (transposed) backward index built only when a backward follows;
 *              the autograd bridge, scale D^-1/2);
 *   [Ascend]   Ascend op-plugin test_npu_block_sparse_attention_backward.py
 *              (BNSD and packed TND layouts, GQA head mapping n / (Hq/Hkv),
 *              per-sequence lengths, the explicit backward taking the forward
 *              output and LSE, the error text for missing TND lengths).
 *
 * Conventions
 *  - Every tensor argument is a DEVICE pointer to a contiguous buffer in the
 *    layout stated below; the caller allocates and owns every buffer (inputs,
 *    outputs, the saved state and the workspace). The library allocates no
 *    device memory and keeps no state between calls; the one exception is the
 *    fixed scratch array that vsa_fwd_noalloc uses in place of a workspace.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *  - Return value: VSA_OK or one of the VSA_ERR_* codes. Argument errors are
 *    detected on the host before anything is launched; vsa_last_error() then
 *    returns a message (thread-local, valid until the next call on the thread).
 *    The compute calls (block_map_to_index, vsa_fwd, vsa_bwd) check every
 *    non-NULL pointer they are given, the problem's valid-count and
 *    cu_seqlens arrays included, with hipPointerGetAttributes: device or
 *    managed memory, or pinned host memory with a device mapping, is accepted;
 *    a plain host pointer gives VSA_ERR_INVALID_ARG ("<name> must be a device
 *    tensor").
 *  - Layouts of q-shaped tensors (q, out, dout, dq, per-element gate):
 *      VSA_BHSD [B, Hq, Sq, D], VSA_BSHD [B, Sq, Hq, D], VSA_TND [Tq, Hq, D];
 *    kv-shaped tensors (k, v, dk, dv) have Hkv heads and Skv (Tkv) rows.
 *    lse is fp32 [B, Hq, Sq] for BHSD and BSHD, [Hq, Tq] for TND.
 *  - Element types: VSA_BF16 or VSA_FP16 for q, k, v, out, dout, gate, dq,
 *    dk, dv, dgate; accumulation is fp32; outputs are rounded to nearest even.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VSA_ABI_VERSION 4

enum vsa_status {
  VSA_OK = 0,
  VSA_ERR_INVALID_ARG = 1, /* bad shape, pointer or combination: nothing launched */
  VSA_ERR_UNSUPPORTED = 2, /* valid request the library has no kernel for        */
  VSA_ERR_WORKSPACE = 3,   /* workspace or saved-state buffer too small          */
  VSA_ERR_HIP = 4          /* a HIP runtime or launch error                      */
};

enum vsa_dtype { VSA_BF16 = 0, VSA_FP16 = 1 };
enum vsa_layout { VSA_BHSD = 0, VSA_BSHD = 1, VSA_TND = 2 };

/* How the compression gate broadcasts ([FV-test] gated test: q-shaped gate;
 * the video workloads: one gate per token and head). */
enum vsa_gate_mode {
  VSA_GATE_NONE = 0,
  VSA_GATE_PER_TOKEN = 1,   /* [B, Hq, Sq] next to BHSD, [B, Sq, Hq] next to BSHD */
  VSA_GATE_PER_ELEMENT = 2, /* q-shaped                                          */
  /* one gate per token and head computed by the library from the token's query
   * row, sigmoid(<q, w_h> + b_h), with learnable parameters gate_proj (see
   * vsa_problem); vsa_fwd writes the gate values to `gate` (per-token layout)
   * when it is not NULL, and vsa_bwd returns their gradient in `dgate` */
  VSA_GATE_PROJECTED = 3
};

/*
 * One attention problem.
 *
 * Sequence geometry ([FV-cute] `_build_vbs_mask_mod`; [Ascend] the golden
 * block expansion): Q rows are cut into blocks of q_block rows and keys into
 * blocks of kv_block keys, counted from the start of each sequence; the last
 * block of a sequence may be partial. Key t of KV block j is live iff
 * (t mod kv_block) < valid(j), where valid(j) is kv_valid[j] when given and
 * never more than the keys that exist in block j. KV blocks with valid(j) == 0
 * are never attended. q_valid only sets the divisor of the pooled Q tiles
 * (the sparse branch computes every existing Q row, padded ones included).
 *
 *   abi_version   must be VSA_ABI_VERSION
 *   dtype, layout see above
 *   B             batch entries (TND: number of sequences)
 *   Hq, Hkv       query heads and key/value heads, Hq % Hkv == 0; Q head h
 *                 reads KV head h / (Hq / Hkv)
 *   Sq, Skv       rows per batch entry (TND: total packed tokens Tq, Tkv)
 *   D             head dimension, 1 .. 128 ([Ascend] page: the operator takes
 *                 head_dim <= 128). The kernels are built for 128; a smaller D
 *                 runs them on copies of the inputs widened with zero columns
 *                 (scores and outputs unchanged, the copies in the caller's
 *                 workspace, results narrowed back), at the cost of D = 128.
 *   q_block       rows per Q block: 8, 16 or a multiple of 32 (8 and 16 run one
 *                 32-row wave per block, with the rows past the block idle)
 *   kv_block      keys per KV block, a multiple of 64
 *   Qb, KVb       blocks per batch entry: ceil(Sq/q_block), ceil(Skv/kv_block)
 *                 (TND: of the longest sequence)
 *   q_valid       device int32 [Qb] valid rows per Q tile, or NULL (= all rows);
 *                 [B, q_valid_batch_stride] with a per-entry stride (below)
 *   kv_valid      device int32 [KVb] valid keys per KV tile, or NULL; likewise
 *   cu_seqlens_q  TND only: device int32 [B+1], exclusive prefix sums of the
 *   cu_seqlens_kv per-sequence lengths (cu[0] = 0, cu[B] = Tq / Tkv)
 *   max_seqlen_q  TND only: the longest q / kv sequence (sizes Qb, KVb)
 *   max_seqlen_kv
 *   scale         softmax scale, > 0 and finite (usually 1/sqrt(D))
 *   topk          0: the caller's block_map is the selection. > 0: select,
 *                 for every Q tile, the topk KV tiles with the largest
 *                 scale * <mean-pooled q, mean-pooled k> (means over valid
 *                 slots; ties to the lower tile; at most the number of
 *                 non-empty tiles). BHSD/BSHD only.
 *   gate_mode     VSA_GATE_NONE, or a compression gate (BHSD/BSHD only):
 *                 out = O_sel + gate * O_c, where O_sel is the sparse-branch
 *                 output and O_c[i] = softmax_j(C[i, j]) V_c[j] is attention
 *                 over the pooled tiles (C as for topk, over all non-empty KV
 *                 tiles), broadcast to every slot of Q tile i.
 *   gate_proj     VSA_GATE_PROJECTED only: device fp32 [Hq * D + Hq], the
 *                 projection weights w ([Hq, D], row h for Q head h) followed
 *                 by the biases b ([Hq]); NULL otherwise
 *   map_batch_stride  elements between batch entries of block_map;
 *                 0 = one [Hq, Qb, KVb] map shared by every batch entry
 *   q_valid_batch_stride, kv_valid_batch_stride  entries between the batch
 *                 entries of q_valid / kv_valid: 0 = one set of counts shared
 *                 by every batch entry (videos of one shape), else at least
 *                 Qb / KVb (a batch of videos with different tile fill, e.g.
 *                 different latent sizes padded to one tile grid; entry b's
 *                 counts start at b * stride). BHSD/BSHD only; the counts
 *                 must then be given.
 *   flags         0, or VSA_FLAG_ATOMIC_DQ: vsa_bwd computes dQ inside the
 *                 KV-owned dK/dV pass (dS K of every selected block added to
 *                 a float accumulator in the backward workspace with atomics,
 *                 then scaled and cast) instead of in a second Q-owned pass
 *                 that recomputes S and dP ([FV-cute] `_build_sparse_tensors`:
 *                 the FA4 backward is KV-owned, one walk per KV tile over the
 *                 query tiles that selected it, so its dQ comes out of that
 *                 same walk). The float sums
 *                 then depend on the order the atomics land in, so dq may
 *                 differ between runs in the last bits; dk, dv and every
 *                 forward output stay bit-reproducible. The default (0) is
 *                 deterministic throughout.
 *                 VSA_FLAG_PERSISTENT, VSA_FLAG_NO_PERSISTENT (either may
 *                 be combined with it): see below.
 */
typedef struct vsa_problem {
  int32_t abi_version;
  int32_t dtype;
  int32_t layout;
  int32_t B, Hq, Hkv;
  int32_t Sq, Skv;
  int32_t D;
  int32_t q_block, kv_block;
  int32_t Qb, KVb;
  const int32_t* q_valid;
  const int32_t* kv_valid;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_kv;
  int32_t max_seqlen_q, max_seqlen_kv;
  float scale;
  int32_t topk;
  int32_t gate_mode;
  int64_t map_batch_stride;
  int32_t flags;
  const float* gate_proj;
  int64_t q_valid_batch_stride;
  int64_t kv_valid_batch_stride;
} vsa_problem;

#define VSA_FLAG_ATOMIC_DQ 1
/* Grid of vsa_bwd's KV-owned dK/dV pass. Persistent: one work-group per
 * compute unit, taking the KV spans from a device list in longest-processing-
 * time order (work estimated from the KV-owned index; ordered by KV head
 * first, then by decreasing work) until none is left. Otherwise: one
 * work-group per span. Results are the same bit for bit either way. By
 * default the persistent grid is used when the pass has at least
 * VSA_PERSISTENT_MIN_SPANS_PER_CU spans per compute unit (the list costs three
 * small extra launches, which pay off only on large problems); these flags
 * force one or the other (setting both is INVALID_ARG). */
#define VSA_FLAG_PERSISTENT 2
#define VSA_FLAG_NO_PERSISTENT 4
#define VSA_PERSISTENT_MIN_SPANS_PER_CU 8

/* Message of the last failed call on this thread ("" after a success). */
const char* vsa_last_error(void);

/* VSA_ABI_VERSION of the built library. */
int vsa_abi_version(void);

/* Host-only check of a problem (no device access). Messages for the cases
 * the pages name: "actual_seq_lengths must be specified",
 * "actual_seq_lengths_kv must be specified" (TND without cu_seqlens_q / _kv).
 * Limits of the library (VSA_ERR_UNSUPPORTED): D <= 128; q_block 8, 16 or a
 * multiple of 32, kv_block a multiple of 64; fewer than 65536 heads in BSHD and
 * TND (row offsets of the tile loads are 24-bit); B*Hq*Qb*KVb and B*Hq*Sq below
 * 2^31; with top-k or a gate, KVb <= 38848 (one row of coarse scores per KV tile
 * in the coarse forward's LDS). */
int vsa_validate(const vsa_problem* p);

/*
 * Host-only sizes, in bytes, of the buffers the caller provides:
 *   ws_fwd       workspace of vsa_fwd (inference and training)
 *   ws_bwd       workspace of vsa_bwd
 *   saved_bytes  state written by a training vsa_fwd and read by vsa_bwd
 *   nnz_capacity upper bound of selected (Q block, KV block) pairs, i.e. the
 *                col capacity block_map_to_index needs for this problem
 * Any output pointer may be NULL.
 */
int vsa_sizes(const vsa_problem* p, size_t* ws_fwd, size_t* ws_bwd, size_t* saved_bytes,
              int64_t* nnz_capacity);

/*
 * Block map -> CSR index of the live (Q block, KV block) pairs
 * ([FV-cute] `_map_to_index`, `_build_sparse_tensors`).
 *   block_map   device uint8 [B, Hq, Qb, KVb] (batch stride p->map_batch_stride);
 *               nonzero = selected
 *   kv_owned    0: rows r = (b*Hq + h)*Qb + i list KV blocks j ascending
 *               1: rows r = (b*Hq + h)*KVb + j list Q blocks i ascending
 *                  (the map transposed: the backward's KV-owned index)
 *   row_ptr     device int32 [rows + 1]: row r is col[row_ptr[r] .. row_ptr[r+1]);
 *               row_ptr[rows] = number of pairs
 *   col_idx     device int32 [col_capacity]
 * A pair is live iff the map entry is nonzero, valid(j) > 0 and (TND) both
 * blocks lie inside sequence b. The result is deterministic. If more than
 * col_capacity pairs are live, row_ptr is still complete and col_idx holds the
 * first col_capacity entries; use vsa_sizes' nnz_capacity to avoid that.
 * ws may be NULL (no workspace is needed).
 */
int block_map_to_index(const vsa_problem* p, const uint8_t* block_map, int kv_owned,
                       int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * Forward ([FV-cute] `_cute_attention`; [FV-test] the VSA entry points).
 *   q, k, v     inputs in the problem layout
 *   block_map   topk == 0: the selection (input).
 *               topk > 0: NULL, or a uint8 [B, Hq, Qb, KVb] buffer that receives
 *               the selection (map_batch_stride must then be Hq*Qb*KVb or 0 with B == 1)
 *   gate        PER_TOKEN / PER_ELEMENT: the gate; PROJECTED: NULL, or a
 *               per-token buffer that receives the gate values; NONE: NULL
 *   out         q-shaped output (the gated output when a gate is given)
 *   lse         fp32 natural-log LSE of the sparse branch; -inf for a row with
 *               no live key (whose output is then 0)
 *   saved       NULL for inference: no backward state is built and out / lse
 *               are bit-identical to a training call ([FV-test] inference test).
 *               Otherwise a buffer of saved_bytes that vsa_bwd reads.
 *   ws          workspace of at least ws_fwd bytes
 */
int vsa_fwd(const vsa_problem* p, const void* q, const void* k, const void* v,
            uint8_t* block_map, const void* gate, void* out, float* lse, void* saved,
            size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);

/*
 * Forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The computation, arguments and results are those of vsa_fwd (out and lse
 * bit for bit), without ws / ws_bytes: the forward workspace is a scratch
 * array of VSA_NOALLOC_SCRATCH_BYTES that the library keeps in each GPU's
 * memory (a static device array, held until the process ends; its device
 * address is looked up on the first call on each device). This call makes no
 * hipMalloc, hipFree or other allocating call and records no profiler events.
 *  - A problem whose forward workspace (ws_fwd of vsa_sizes) exceeds
 *    VSA_NOALLOC_SCRATCH_BYTES gives VSA_ERR_WORKSPACE before any launch.
 *  - stream must belong to the current device (else VSA_ERR_INVALID_ARG).
 *  - Every call on one GPU uses that GPU's single scratch: calls that overlap
 *    on one GPU (other streams, other threads) race and must be serialised by
 *    the caller. Nothing in the scratch needs to start at zero: each call
 *    writes every part of it that it reads.
 *  - saved (training) is still a caller buffer, as for vsa_fwd.
 */
#define VSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int vsa_fwd_noalloc(const vsa_problem* p, const void* q, const void* k, const void* v,
                    uint8_t* block_map, const void* gate, void* out, float* lse, void* saved,
                    size_t saved_bytes, void* stream);

/*
 * Backward of L = sum(out * dout) ([FV-cute] `_CuteAttentionQ128.backward`;
 * [Ascend] the explicit backward golden): recomputes P from lse, uses the row
 * term rowsum(dout * O_sel), dQ from the Q-owned index and dK / dV from the
 * KV-owned index without atomics, dK / dV summed over the Q heads of each KV
 * head. With a gate, the compression branch adds its pooled gradients (valid
 * slots only) and dgate (optional) receives dL/dgate. No gradient flows
 * through the top-k choice. Rows whose q and dout are both zero (the padded
 * slots of video tiles in training) have dS = 0 and are skipped; for finite
 * inputs the results are those of the full computation.
 *   q, k, v, gate  the forward's inputs (PROJECTED: gate is not read)
 *   dout        q-shaped upstream gradient; NULL means zeros
 *   out         the forward's output (read only when gate_mode == NONE; with a
 *               gate the un-gated sparse output kept in `saved` is used)
 *   lse         the forward's lse
 *   saved       the buffer a training vsa_fwd filled
 *   dq          q-shaped; dk, dv kv-shaped (Hkv heads); dgate gate-shaped or
 *               NULL (PROJECTED: fp32 [Hq * D + Hq], the gradient of gate_proj;
 *               the projection's own term dL/dz w_h is part of dq)
 *   ws          workspace of at least ws_bwd bytes
 */
int vsa_bwd(const vsa_problem* p, const void* q, const void* k, const void* v, const void* gate,
            const void* dout, const void* out, const float* lse, const void* saved,
            size_t saved_bytes, void* dq, void* dk, void* dv, void* dgate, void* ws,
            size_t ws_bytes, void* stream);

/*
 * Opt-in per-kernel timing (instrumentation, not needed for computing).
 * Between vsa_profile_begin() and vsa_profile_end() the library records a
 * pair of HIP events around each of its kernel launches, on the launch
 * stream. vsa_profile_end() waits for those events and writes, for every
 * kernel id k < n, the summed duration in milliseconds (ms_total[k]) and the
 * number of launches (launches[k]). Recording stops silently after 65536
 * launches. Process-wide state: do not profile from several threads at once.
 */
enum vsa_kernel_id {
  VSA_KERNEL_INDEX = 0,       /* block map -> CSR (count, scan, fill) */
  VSA_KERNEL_POOL = 1,        /* mean-pooled tiles                    */
  VSA_KERNEL_COARSE_FWD = 2,  /* coarse scores, top-k, coarse attention */
  VSA_KERNEL_SPARSE_FWD = 3,  /* sparse-branch forward                */
  VSA_KERNEL_BWD_PRE = 4,     /* row term rowsum(dO * O_sel), gate sums */
  VSA_KERNEL_COARSE_BWD = 5,  /* compression-branch backward          */
  VSA_KERNEL_SPARSE_DKDV = 6, /* KV-owned dK / dV                     */
  VSA_KERNEL_SPARSE_DQ = 7,   /* Q-owned dQ                           */
  VSA_KERNEL_DQ_ATOMIC = 8,   /* atomic-dQ backward: accumulator clear and cast */
  VSA_KERNEL_DKDV_ORDER = 9,  /* persistent dK/dV grid: the longest-first span list */
  VSA_KERNEL_PAD = 10,        /* D < 128: widening inputs, narrowing results */
  VSA_KERNEL_COUNT = 11
};

int vsa_profile_begin(void);
int vsa_profile_end(double* ms_total, int64_t* launches, int n);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */
