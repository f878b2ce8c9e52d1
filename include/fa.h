/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * The library computes exact (not approximate) softmax attention
 *
 *     O = softmax(scale * Q K^T + causal mask) V,   LSE_i = ln sum_j exp(scale * q_i . k_j)
 *
 * the way FlashAttention-2 organises it: one workgroup per query tile, key
 * and value tiles streamed through LDS, an online softmax (running row max
 * and row sum, rescaled as the max grows), the output accumulator kept in
 * registers, and tiles above the causal diagonal skipped.  Sources:
 *   - scores S = Q K^T / sqrt(d) and P = exp(S - m) / l:
 *     "Adaptive High-Performance Attention Kernels in CUDA", Advanced
 *     Production Features, 2. Custom CUDA Backward Pass;
 *   - the running max / running sum recurrence: "FlashAttention-2 MMA",
 *     Technical Details, Online Softmax (Safe Softmax);
 *   - the causal rule key index <= query index: "FlashAttention-2 MMA",
 *     Technical Details, Causal Masking;
 *   - split-KV decoding (partial attention over key partitions, then a
 *     log-sum-exp merge): "Adaptive High-Performance Attention Kernels in
 *     CUDA", Advanced Production Features, 1. Split-K FlashDecoding, and
 *     "FlashAttention-2 MMA", Supported Dispatch Strategies (Split-KV).
 *
 * Conventions shared by every entry point
 *   Tensors   q, k, v, o are IEEE fp16, contiguous row-major [B, H, S, D]
 *             (D innermost, then sequence, then head, then batch).  q and o
 *             have S = Sq, k and v have S = Sk.  lse is fp32 [B, H, Sq].
 *   Memory    every tensor pointer is device memory owned by the caller and
 *             must stay valid until the stream has executed the call.
 *             q, k, v, o must be 16-byte aligned, lse 4-byte aligned.  The
 *             library keeps no pointer after it returns and never frees or
 *             synchronises caller memory.
 *   Stream    `stream` is a hipStream_t passed as void* (NULL = the null
 *             stream).  Every call only enqueues work on that stream and
 *             returns; results are valid once the stream has reached them.
 *             No call waits on the host or makes one stream wait for another.
 *   Causal    top-left aligned: query row i sees keys 0..i (all keys when
 *             i >= Sk), so no row is ever fully masked.
 *   Scale     any finite scale > 0 (the pages use 1/sqrt(D)).
 *   Limits    one [S, D] slice of q, k, v or o must stay below 2 GiB
 *             (S * D * 2 < 2^31 bytes); the tensors as a whole may be larger.
 *   LSE       natural logarithm of the row sum of exp(scale * q . k) over the
 *             visible keys.
 *   Errors    a non-zero return is one of the FA_ERR_* codes.  Arguments are
 *             validated on the host before any HIP call, so an invalid call
 *             enqueues nothing.  FA_ERR_HIP reports a failed HIP launch or
 *             allocation; fa_last_error() then names it.
 *   Threads   the library's only state is a per-device CU count cache, a
 *             per-device stream-ordered workspace memory pool (created once,
 *             under a lock) and a thread-local error message; calls share no
 *             buffer with each other and may be made from several threads
 *             and on several streams at once.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, size out of range, bad scale, ... */
  FA_ERR_UNSUPPORTED = 2, /* head dim not supported by the entry point */
  FA_ERR_HIP = 3          /* a HIP call or kernel launch failed */
};

/*
 * fa_fwd -- exact attention forward (prefill), FlashAttention-2 style.
 *
 *   q      [B, H, Sq, D] fp16        k, v  [B, H, Sk, D] fp16
 *   o      [B, H, Sq, D] fp16 out    lse   [B, H, Sq]    fp32 out
 *   B, H, Sq, Sk >= 1;  D in {32, 64, 128, 256, 512, 1024};  causal 0 or 1;
 *   scale > 0.
 *
 * Queries are split into tiles, one workgroup each ("Split-Q" in
 * "FlashAttention-2 MMA", Supported Dispatch Strategies; loop order of
 * "Adaptive High-Performance Attention Kernels in CUDA", Architectural
 * Progression, Stage 3).  With causal = 1 the key tiles that lie wholly
 * above the diagonal are never loaded (same page, Lever A).  Head dims 512
 * and 1024 take the Split-D kernel (same strategy list, 3. Split-D): the
 * D/128 wavefronts of a workgroup share 32 query rows, each owns a 128-wide
 * slice of D, and their partial scores are summed through LDS.  When those
 * (query tile, slice) work items are fewer than the CUs, the Split-D key
 * range is also split and the parts merged with log-sum-exp weights
 * ("Split-KV" of the same list).  A grid of at most two query tiles per CU
 * whose heaviest query tiles would leave most CUs idle near the end has key
 * ranges split, when fa_fwd_key_splits() says it pays: causal grids at D <=
 * 128 too small for 256-row workgroups split the key ranges of their
 * heaviest tiles into equal parts; at D = 256 the key tiles of all query
 * tiles are cut into one run per CU (a tile cut between runs is processed
 * in parts).  A second kernel merges the parts.  Split calls keep their fp32 partials in
 * a workspace of fa_fwd_workspace_bytes() bytes taken from the per-device
 * stream-ordered pool (hipMallocFromPoolAsync before the kernels,
 * hipFreeAsync after them, both on `stream`), so nothing blocks and calls on
 * different streams never share a buffer; fa_fwd_ws is the same call with a
 * caller-owned workspace.
 * Any Sq works.  A non-causal call with Sq = 1 and D <= 256 is a decode step
 * and runs fa_decode_splitkv with the automatic split count (the page's
 * dispatch of seq_q == 1 to Split-KV); with causal = 1 a single row sees
 * key 0 only and stays on the prefill kernel.  o and lse must not overlap
 * the inputs.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Sq, int Sk, int D, int causal, float scale,
           void* stream);

/*
 * fa_fwd_workspace_bytes -- bytes of device workspace that fa_fwd (from its
 * pool) and fa_fwd_ws (from the caller) use for these sizes on a device with
 * num_cus CUs: 0 when the call runs without one (no key split, and a decode
 * step with one partition); otherwise the fp32 partial outputs and LSEs of
 * the key parts, rows * parts * (D + 1) * 4 bytes rounded up to 256, where
 * rows are the query rows of the split tiles (B * H * Sq for Split-D, and
 * B * H for a decode step); at D = 256, two 128-row slots of partial O and
 * LSE per run, each of the two arrays rounded up to 256.  Pure host
 * arithmetic; returns 0 for invalid sizes too.
 */
size_t fa_fwd_workspace_bytes(int B, int H, int Sq, int Sk, int D, int causal, int num_cus);

/*
 * fa_fwd_ws -- fa_fwd with a caller-provided device workspace: at least
 * fa_fwd_workspace_bytes(B, H, Sq, Sk, D, causal, CUs of the current device)
 * bytes, 16-byte aligned; it may be NULL when that is 0.  Nothing is
 * allocated.  Same computation, kernels, stream behaviour and results as
 * fa_fwd.  A smaller workspace returns FA_ERR_INVALID_ARG before any launch.
 * Calls that share one workspace must be ordered on one stream (or
 * otherwise serialised by the caller); the workspace holds no result.
 */
int fa_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Sq, int Sk, int D, int causal, float scale,
              void* stream, void* workspace, size_t workspace_bytes);

/*
 * fa_bwd -- gradients of exact attention from the forward's outputs
 * ("Adaptive High-Performance Attention Kernels in CUDA", Advanced
 * Production Features, 2. Custom CUDA Backward Pass: S and P recomputed
 * from the forward statistics, D_i = sum_d dO_id O_id, dS = P o (dP - D)).
 *
 *   q, k, v, o, lse  as passed to / returned by fa_fwd with the same B, H,
 *                    Sq, Sk, D, causal and scale (lse: natural log)
 *   dout             fp16 [B, H, Sq, D], the gradient of the loss w.r.t. o
 *   dq               fp16 [B, H, Sq, D]  = scale * dS K
 *   dk, dv           fp16 [B, H, Sk, D]  dk = scale * dS^T Q, dv = P^T dO
 * with P = exp(scale * Q K^T + mask - lse), dP = dout V^T.  All tensors are
 * caller-owned device memory, 16-byte aligned (lse 4-byte); outputs must not
 * overlap inputs.  A per-row workspace (D and the LSE in log2 units,
 * fa_bwd_workspace_bytes) comes from the same per-device pool as
 * fa_decode_splitkv.  Two kernels run on `stream`: dQ, which also forms D_i
 * and the log2 LSE of every query row into the workspace, then dK and dV
 * (each kernel forms S, P, dP and dS of its own tiles, so no partial sums
 * cross workgroups and the result is bitwise repeatable).  Supports D in {32, 64, 128, 256} (other D:
 * FA_ERR_UNSUPPORTED); other errors as fa_fwd.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D,
           int causal, float scale, void* stream);

/*
 * fa_bwd_workspace_bytes -- device workspace of fa_bwd / fa_bwd_ws: one fp32
 * D and one fp32 LSE (log2 units) per query row, 2 * B * H * Sq * 4 bytes
 * rounded up to 256.  Pure host arithmetic; 0 for invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Sq, int D);

/*
 * fa_bwd_ws -- fa_bwd with a caller-provided device workspace of at least
 * fa_bwd_workspace_bytes(B, H, Sq, D) bytes, 16-byte aligned (a null,
 * misaligned or smaller one returns FA_ERR_INVALID_ARG before any launch).
 * Nothing is allocated; same kernels and results as fa_bwd.  Calls that
 * share one workspace must be ordered on one stream; the workspace holds no
 * result.
 */
int fa_bwd_ws(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D,
              int causal, float scale, void* stream, void* workspace, size_t workspace_bytes);

/*
 * fa_fwd_varlen -- fa_fwd over a packed batch of variable-length sequences
 * ("Adaptive High-Performance Attention Kernels in CUDA", Advanced
 * Production Features, 3. Ragged / Variable-Length Sequences: one token
 * stream [total_tokens, H, d] indexed by cumulative sequence lengths, no
 * padding).
 *
 *   q, o          fp16 [total_q, H, D], 16-byte aligned
 *   k, v          fp16 [total_k, H, D], 16-byte aligned
 *   lse           fp32 [H, total_q], 4-byte aligned
 *   cu_seqlens_q  int32 [B + 1] device memory: sequence b owns query tokens
 *   cu_seqlens_k  cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key tokens
 *                 cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 (4-byte aligned)
 *   max_seqlen_q  upper bounds of the per-sequence lengths; the grid covers
 *   max_seqlen_k  max_seqlen_q query rows per sequence and head
 * Within each sequence the computation is fa_fwd's (causal = top-left
 * aligned: query i of a sequence sees its keys 0..i).  Device-side values
 * are not trusted: each start is clamped to [0, total] and each length to
 * [0, min(total - start, max_seqlen)], so nothing outside the tensors is
 * read or written.  Query rows that no sequence covers are left untouched;
 * a query row whose sequence has no key gets o = 0 and lse = -inf.
 * D in {32, 64, 128, 256} (other D: FA_ERR_UNSUPPORTED).
 * Limits: (max_seqlen + 256) * H * D * 2 < 2^31 bytes for q and for k.
 * Errors as fa_fwd.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                  int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int D,
                  int causal, float scale, void* stream);

/*
 * fa_decode_splitkv -- single-query decoding with the key range split into
 * num_splits contiguous partitions ("Adaptive High-Performance Attention
 * Kernels in CUDA", Advanced Production Features, 1. Split-K FlashDecoding).
 *
 * Same arguments as fa_fwd plus num_splits; requires Sq == 1 and causal == 0
 * (FA_ERR_INVALID_ARG otherwise) and D in {32, 64, 128, 256}
 * (FA_ERR_UNSUPPORTED otherwise).  Partition s covers keys
 * [s*c, min((s+1)*c, Sk)) with c = ceil(Sk / num_splits); trailing
 * partitions may be empty.  num_splits <= 0 picks fa_decode_auto_splits()
 * for the current device; otherwise 1 <= num_splits <= Sk.
 * With one partition (num_splits == 1), one 1024-thread workgroup per
 * (batch, head) splits the keys over its 16 wavefronts, merges their
 * partial states in LDS with the same log-sum-exp weights and writes o and
 * lse: one kernel, no workspace.  Otherwise phase one writes a normalised
 * partial output and its LSE per partition, and phase two merges them with
 * log-sum-exp weights into o and lse.  Both kernels run on `stream`.  The partials live in a workspace taken from a
 * per-device memory pool that the library creates on first use (stream-
 * ordered hipMallocFromPoolAsync / hipFreeAsync on `stream`, so nothing
 * blocks); the pool keeps freed memory for reuse until the process ends.
 */
int fa_decode_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Sq, int Sk, int D, int causal, float scale,
                      void* stream, int num_splits);

/*
 * fa_decode_workspace_bytes -- bytes of workspace fa_decode_splitkv_ws needs
 * for these sizes: B*H*num_splits*(D + 1) fp32 values, rounded up to 256.
 * num_splits must be >= 1 (use fa_decode_auto_splits first for "auto").
 * Returns 0 for invalid sizes.
 */
size_t fa_decode_workspace_bytes(int B, int H, int D, int num_splits);

/*
 * fa_decode_splitkv_ws -- fa_decode_splitkv with a caller-provided device
 * workspace (at least fa_decode_workspace_bytes(B, H, D, ns) bytes, 16-byte
 * aligned, where ns is the resolved split count).  Nothing is allocated.
 * On return the workspace is laid out as partial outputs fp32
 * [B, H, ns, D] followed by partial LSEs fp32 [B, H, ns] (natural log;
 * -inf for an empty partition, whose partial output is 0).  With ns == 1
 * the workspace is checked but not touched.  Calls that share one
 * workspace must be ordered on one stream.
 */
int fa_decode_splitkv_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int Sq, int Sk, int D, int causal, float scale,
                         void* stream, int num_splits, void* workspace, size_t workspace_bytes);

/*
 * fa_decode_splitkv_noalloc -- fa_decode_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): same arguments, same kernels and
 * bit-identical results for the same resolved split count.  It calls no
 * allocator.  With more than one partition the phase-one partials live in
 * a static scratch array of 16 MiB (16777216 bytes) that the library's
 * code object holds on every GPU it runs on until the process ends; a call
 * whose partials, B*H*ns*(D + 1)*4 bytes rounded up to 256, exceed it
 * returns FA_ERR_INVALID_ARG before any launch.  Every call on one GPU
 * shares that GPU's scratch (its contents are whatever the last call left;
 * phase one overwrites every partial it merges, so nothing needs
 * clearing): calls that may overlap on one GPU -- on different streams, or
 * from different threads -- race and must be serialised by the caller.
 */
int fa_decode_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int Sq, int Sk, int D, int causal, float scale,
                              void* stream, int num_splits);

/*
 * fa_decode_paged -- fa_decode_splitkv over a paged KV cache ("Adaptive
 * High-Performance Attention Kernels in CUDA", Advanced Production
 * Features, 4. PagedAttention: physical pages [num_blocks, H, block_size, D]
 * and a block table translating logical token positions to pages).
 *
 *   q, o          fp16 [B, H, 1, D]; lse fp32 [B, H, 1] (16- / 4-byte aligned)
 *   k_cache,      fp16 [num_blocks, H, block_size, D], 16-byte aligned
 *   v_cache
 *   block_tables  int32 [B, max_blocks] device memory: entry (b, j) is the
 *                 physical block holding keys j*block_size .. +block_size-1
 *                 of sequence b (4-byte aligned)
 *   seq_lens      int32 [B] device memory: context length of each sequence
 *   block_size    a power of two, 1 .. 1024
 * Sequence b attends, non-causally, to its keys 0 .. seq_lens[b]-1, split
 * into num_splits partitions of ceil(seq_lens[b] / num_splits) keys as in
 * fa_decode_splitkv.  Device-side values are not trusted: seq_lens[b] is
 * clamped to [0, max_blocks * block_size], a table entry outside
 * [0, num_blocks) marks its keys absent (they are never read and do not
 * count), and a sequence with no present key gets o = 0 and lse = -inf.
 * num_splits <= 0 picks fa_decode_auto_splits(B, H, max_blocks *
 * block_size, CUs); otherwise 1 <= num_splits <= max_blocks * block_size.
 * At equal num_splits the result is bit-identical to fa_decode_splitkv on
 * the same keys held contiguously (the keys are visited in the same order).
 * Workspace, pool and stream behaviour as fa_decode_splitkv.  Returns
 * FA_ERR_INVALID_ARG for null / misaligned pointers or bad sizes,
 * FA_ERR_UNSUPPORTED for D not in {32, 64, 128, 256}.
 */
int fa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                    const int* block_tables, const int* seq_lens, void* o, float* lse,
                    int B, int H, int D, int num_blocks, int block_size, int max_blocks,
                    float scale, void* stream, int num_splits);

/*
 * fa_decode_auto_splits -- the split count fa_decode_splitkv uses when
 * num_splits <= 0: 1 when B*H >= 2 * num_cus (one 1024-thread workgroup
 * per slice then gives every CU two); otherwise the smallest power of two
 * that gives at least 8 * num_cus 256-thread phase-one workgroups, lowered
 * until every partition holds at least 256 keys (never below 1, never above
 * Sk).  Pure host arithmetic; returns 0 for invalid sizes.
 */
int fa_decode_auto_splits(int B, int H, int Sk, int num_cus);

/*
 * fa_fwd_key_splits -- the most key-range parts into which fa_fwd cuts any
 * query tile of these sizes on a device with num_cus CUs (1: no split), the
 * same plan fa_fwd makes ("Adaptive High-Performance Attention Kernels in
 * CUDA", Split-K / Flash-Decoding, applied to prefill query tiles).  Causal
 * D = 32, 64, 128 grids of 128-row workgroups (those with fewer 256-row
 * tiles than CUs): the parts of the heaviest tiles, chosen by simulating
 * the dispatch of the work items (heaviest first, each to the CU that frees
 * first) against the cost of merging the parts.  D = 256 grids of at most
 * two query tiles per CU: one run of key tiles per CU, chosen by modelling
 * each run's segments against the unsplit grid and the merge.  Timing
 * constants are measured per kernel; at most 8 parts.  Other D = 64, 128
 * grids: 1.  D = 512, 1024: the Split-D key split (enough parts to give
 * every CU a work item when there are fewer than CUs, at most 16).  A
 * decode step (Sq = 1, causal = 0, D <= 256): the partitions of
 * fa_decode_auto_splits.  Pure host arithmetic; returns 0 for invalid sizes.
 */
int fa_fwd_key_splits(int B, int H, int Sq, int Sk, int D, int causal, int num_cus);

/* fa_status_string -- static text for an FA_* status code. */
const char* fa_status_string(int status);

/* fa_last_error -- text of the last FA_ERR_* raised on this thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
