/*
 * fa.h -- C ABI of the exact, IO-aware attention library (libfa.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed
 *   Exact scaled-dot-product attention and its gradient, never writing the
 *   N x N score matrix to device memory:
 *     S = (Q K^T) * scale, masked entries -inf, P = softmax_row(S), O = P V,
 *     lse_i = ln sum_j exp(S_ij).
 *   The pages this follows: "[Paper Review] FlashAttention-2: Faster
 *   Attention with Better Parallelism and Work Partitioning" (nubint.ai;
 *   Abstract, "Proposed method") for exactness, the online-softmax tiling,
 *   parallelism over sequence length and causal block skipping; and
 *   "Researchers at Stanford University Propose FlashAttention: Fast and
 *   Memory-Efficient Exact Attention with IO-Awareness" for keeping the
 *   attention matrix out of HBM, saving the softmax normalisation statistic
 *   (lse) in the forward and recomputing attention on chip in the backward,
 *   and block-sparse attention.
 *
 * Conventions shared by every entry point
 *   - q, k, v, o, dO, dq, dk, dv: device pointers to bfloat16 bit patterns
 *     (uint16_t), contiguous [B][H][N][d] (d fastest). d must be 64 or 128.
 *     Device pointers must be 16-byte aligned.
 *   - lse: device pointer, float32 [B][H][N], natural-log logsumexp of the
 *     scaled, masked score row; -inf for a row that sees no key.
 *   - One sequence length N for queries and keys. causal != 0 makes key j
 *     visible from query i only when j <= i.
 *   - scale: finite and > 0 (callers normally pass 1/sqrt(d)).
 *   - block_mask: device pointer, uint8 [H][nb][nb] with nb = ceil(N/128);
 *     nonzero keeps the 128 x 128 block (query block, key block), shared by
 *     every batch entry. With causal, a pair must pass both.
 *   - stream: a hipStream_t (e.g. torch.cuda.current_stream().cuda_stream),
 *     or NULL for the default stream. Work is only enqueued; nothing waits
 *     on the host. Outputs must not alias inputs.
 *   - Ownership: the caller allocates and frees every buffer, including the
 *     backward workspace. The library keeps no device memory of its own and
 *     no state that changes results. Per-process state it does keep: each
 *     kernel's occupancy (workgroups per CU, asked of the runtime on the
 *     first launch and cached, used only to pick the launch order of causal
 *     and block-sparse grids) and, for fa_std_fwd, one rocBLAS handle per
 *     device.
 *   - Errors: every entry point returns FA_OK (0) or a negative fa_status.
 *     Argument checks run before anything is enqueued; a failed launch is
 *     reported as FA_ERR_HIP. Faults during execution surface at the
 *     caller's next synchronisation of the stream.
 *   - Output rounding: o, dq, dk, dv are rounded to bfloat16 to nearest-even
 *     from float32 accumulators.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = -1,           /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,          /* B, H or N < 1, or B*H*N*d too large */
    FA_ERR_UNSUPPORTED_D = -3,  /* d not in {64, 128} */
    FA_ERR_SCALE = -4,          /* scale not finite or <= 0 */
    FA_ERR_WORKSPACE = -5,      /* backward workspace missing or too small */
    FA_ERR_MASK = -6,           /* block_mask NULL in a block-sparse call */
    FA_ERR_HIP = -7,            /* a HIP launch, runtime or rocBLAS call failed */
    FA_ERR_ALIGN = -8,          /* a pointer is not 16-byte aligned */
    FA_ERR_DROPOUT = -9         /* dropout probability not in [0, 1) */
} fa_status;

/* Forward. Writes o [B][H][N][d] (bf16) and lse [B][H][N] (fp32).
 * One workgroup per (batch, head, query tile); key/value tiles are streamed
 * through LDS with an online softmax (FlashAttention-2 review, "Proposed
 * method"; Stanford FlashAttention summary, tiling and incremental softmax). */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, int causal, float scale, void* stream);

/* Forward with a 128 x 128 block mask; masked blocks are skipped entirely
 * (Stanford FlashAttention summary, block-sparse FlashAttention). */
int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, int causal, float scale,
                       const uint8_t* block_mask, void* stream);

/* Forward with an explicit tile configuration, for tile-size studies (the
 * IO analysis of the Stanford FlashAttention summary: HBM accesses against
 * on-chip memory size). Same computation and arguments as
 * fa_fwd_blocksparse (block_mask may be NULL for dense), plus
 *   bm: query rows per workgroup (128: 4 waves, two workgroups per CU;
 *       256: 8 waves, one workgroup per CU),
 *   bn: keys per K/V tile staged in LDS.
 * Supported (bm, bn): (128, 32), (128, 64), (128, 128), (256, 64),
 * (256, 128); any other pair returns FA_ERR_SHAPE. fa_fwd and
 * fa_fwd_dropout use (128, 32) at d = 128 and (128, 64) at d = 64. */
int fa_fwd_tiles(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, int causal, float scale,
                 const uint8_t* block_mask, int bm, int bn, void* stream);

/* Standard attention, for comparison: the computation FlashAttention
 * replaces, with the N x N score matrix written to and read back from device
 * memory (Stanford FlashAttention summary, the paragraph on reads and writes
 * of the attention matrix; FlashAttention-2 review, Abstract: memory
 * quadratic in sequence length). Same arguments, results and conventions as
 * fa_fwd_blocksparse (block_mask may be NULL for dense), plus a workspace of
 * fa_std_workspace_size bytes (fp32 S and bf16 P, 6 * B * H * N * N bytes).
 * S = Q K^T * scale and O = P V are rocBLAS strided-batched GEMMs (bf16
 * operands, fp32 accumulation); masking and the row softmax are a HIP kernel.
 * N <= 16384. The library keeps one rocBLAS handle per device for the life
 * of the process. Library failures are reported as FA_ERR_HIP. */
int fa_std_workspace_size(int B, int H, int N, int d, size_t* bytes);
int fa_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, int causal, float scale,
               const uint8_t* block_mask, void* workspace, size_t workspace_bytes, void* stream);

/* FlashAttention-1-style forward, kept as a measured ablation of the
 * FlashAttention-2 changes (FlashAttention-2 review, Abstract items (1)-(3)
 * and "Research questions", RQ2): one workgroup per (batch, head) with no
 * parallelism over sequence length; K/V tiles in the outer loop and query
 * tiles in the inner loop, the running output, max and sum of every row
 * kept in a device workspace and read and written back once per K/V tile;
 * the keys of a tile split across the waves, combined through LDS; the
 * output normalised after every tile. Same arguments and results as fa_fwd
 * (no block mask), plus:
 *   seq_groups  1 reproduces the published partitioning (B*H workgroups).
 *               G > 1 deals the head's 32-row query tiles round-robin to G
 *               workgroups per head (clamped to ceil(N/32)), adding only the
 *               sequence parallelism of FlashAttention-2, so that its effect
 *               is measured apart from the other two changes. < 1:
 *               FA_ERR_SHAPE.
 *   workspace   fa_fa1_workspace_size bytes of device memory, 16-byte
 *               aligned, owned by the caller (fp32 output and per-wave
 *               max/sum rows, linear in N); too small or NULL:
 *               FA_ERR_WORKSPACE. Contents on entry are ignored. */
int fa_fa1_workspace_size(int B, int H, int N, int d, size_t* bytes);
int fa_fwd_fa1(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, int causal, float scale, int seq_groups,
               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace fa_bwd / fa_bwd_blocksparse need, O(B*H*N) --
 * never O(N^2) (FlashAttention-2 review, Abstract: memory linear instead of
 * quadratic in sequence length; Stanford FlashAttention summary: only the
 * softmax normalisation statistic is kept for the backward pass):
 * float32 D = rowsum(dO * O) and lse * log2(e) for every row
 * (rows padded to 128 per head), then, for block-sparse calls, a schedule of
 * three int32 per (head, 128-row mask block): the key and query tiles of
 * each head in order of falling work, which the schedule stage writes
 * (masks of more than 2048 blocks per row keep the plain order). The order
 * changes only which tiles run first, never the results. */
int fa_bwd_workspace_size(int B, int H, int N, int d, size_t* bytes);

/* Backward. Inputs: q, k, v, the forward's o and lse, and the upstream
 * gradient dO. Writes dq, dk, dv (bf16, [B][H][N][d]). Attention
 * probabilities are recomputed on chip from lse (Stanford FlashAttention
 * summary, recomputation in the backward pass). Two kernels on `stream`:
 * dQ parallel over query tiles, which also writes D = rowsum(dO*O) and
 * lse * log2(e) per row into the workspace; then dK/dV parallel over key
 * tiles, which reads them. Deterministic (no atomics). */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, int causal, float scale,
           void* workspace, size_t workspace_bytes, void* stream);

/* Backward with a 128 x 128 block mask (same convention as the forward);
 * masked blocks are skipped in both backward kernels (Stanford
 * FlashAttention summary, block-sparse FlashAttention). */
int fa_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dO, void* dq, void* dk, void* dv,
                       int B, int H, int N, int d, int causal, float scale,
                       const uint8_t* block_mask,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Backward that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same computation, arguments and results as
 * fa_bwd_blocksparse (block_mask NULL for dense attention), without the
 * workspace arguments: the scratch the backward needs (fa_bwd_workspace_size
 * bytes) lives in one device array of 16 MiB inside the library, which each
 * GPU the library runs on holds until the process ends. Sizes whose
 * fa_bwd_workspace_size exceeds 16 MiB (about B*H*ceil(N/128)*128 > 2
 * million rows) return FA_ERR_WORKSPACE before anything is enqueued. The
 * call makes no hipMalloc, hipFree or other allocation; its first call on a
 * device looks up that device's array address once. Every call on one GPU
 * shares that GPU's array, and nothing needs to start at zero (each call
 * writes the scratch before reading it), but calls that overlap in time on
 * one GPU (on different streams, or from several host threads without
 * ordering) race on it and give wrong results. */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, int causal, float scale,
                   const uint8_t* block_mask, void* stream);

/* One backward kernel alone, so a caller can time or overlap them (the
 * three steps of the backward pass that recomputes attention on chip,
 * Stanford FlashAttention summary, recomputation; the dK/dV and dQ steps
 * are parallel over sequence length, FlashAttention-2 review, "Proposed
 * method"); fa_bwd
 * (fa_bwd_blocksparse when block_mask != NULL) is exactly stages 0, 1, 2
 * enqueued in that order on one stream. stage 0: with a block mask, the
 * schedule of tiles by falling work into the workspace (reads block_mask);
 * without one it enqueues nothing. stage 1: dQ, and D = rowsum(dO * O) and
 * lse * log2(e) per row into the workspace (reads q, k, v, o, lse, dO and
 * the schedule). stage 2: dK and dV (reads q, k, v, dO and the workspace
 * written by stages 0 and 1). Every pointer argument is validated as in
 * fa_bwd whatever the stage. A stage outside 0..2 returns FA_ERR_SHAPE. */
int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dO, void* dq, void* dk, void* dv,
                 int B, int H, int N, int d, int causal, float scale,
                 const uint8_t* block_mask,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Attention dropout (the "PagedAttention" page lists dropout among
 * attention's O(N^2) elementwise operations and defines nothing more; the
 * semantics below are this library's reading). Dropout acts on the
 * normalised probabilities before they multiply V:
 *   O = (P o Z) V / (1 - p),   lse unchanged (that of the undropped row),
 * with Z_ij in {0, 1} regenerated inside the kernels from a counter-based
 * generator, Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011), so no mask is stored:
 *   word j % 4 of Philox4x32-10(counter (j / 4, i, b*H + h, offset),
 *                                key (seed mod 2^32, seed / 2^32))
 * keeps key j of query row i iff it is >= floor(p * 2^32).
 * The backward is the gradient with Z held fixed (same seed and offset as
 * the forward): dV = (P o Z)^T dO / (1 - p), dP = (dO V^T) o Z / (1 - p),
 * D = rowsum(dO o O), dS = P o (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 * Arguments as fa_fwd / fa_bwd, with block_mask NULL for dense attention,
 * plus dropout_p in [0, 1) (else FA_ERR_DROPOUT), seed and offset. Default
 * tile configuration only. */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale,
                   const uint8_t* block_mask, float dropout_p, uint64_t seed,
                   uint32_t offset, void* stream);
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, int causal, float scale,
                   const uint8_t* block_mask, float dropout_p, uint64_t seed,
                   uint32_t offset, void* workspace, size_t workspace_bytes,
                   void* stream);
/* The keep mask Z of the same generator, one byte (0 or 1) per element into
 * keep, a device buffer uint8 [B][H][N][N] owned by the caller (tests of
 * the generator; O(N^2) memory). The "PagedAttention" page names dropout
 * only; the generator and its counter layout are this library's reading
 * (Philox4x32-10, see fa_fwd_dropout). */
int fa_dropout_keep(int B, int H, int N, float dropout_p, uint64_t seed,
                    uint32_t offset, uint8_t* keep, void* stream);

/* Tile sizes the kernels use, so a caller can size the visit maps below.
 * A utility of this library: no passage of the pages defines it (they fix
 * no tile sizes). Returns FA_ERR_UNSUPPORTED_D for d not in {64, 128},
 * FA_ERR_SHAPE for a pass outside 0..2, FA_ERR_NULL for a NULL output.
 * pass: 0 = forward (every forward entry point but fa_fwd_tiles), 1 =
 * backward dK/dV kernel, 2 = backward dQ kernel; causal: nonzero for the causal kernels
 * (the d = 128 dQ kernel streams 64-key tiles when causal, 32-key tiles
 * otherwise). bm = query rows per tile, bn = key rows per tile. */
int fa_tile_config(int pass, int d, int causal, int* bm, int* bn);

/* Debug forward: same computation as fa_fwd_blocksparse (block_mask may be
 * NULL for dense) and additionally writes which tiles were skipped, so the
 * skip decisions can be checked bit for bit: whole key tiles past the
 * diagonal under causal masking (FlashAttention-2 review, "Proposed
 * method": blocks that causal masking zeroes are not computed) and masked
 * blocks of a block-sparse mask (Stanford FlashAttention summary,
 * block-sparse FlashAttention: masked blocks are skipped). It writes visited, uint8
 * [B][H][ceil(N/bm)][ceil(N/bn)] (pass 0 tile sizes): 1 where the kernel
 * processed the (query tile, key tile) pair, 0 where it skipped it. The
 * caller zeroes `visited` before the call. */
int fa_fwd_debug_visits(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int N, int d, int causal, float scale,
                        const uint8_t* block_mask, uint8_t* visited, void* stream);

/* Debug backward: same computation as fa_bwd_blocksparse (block_mask may be
 * NULL), with the skip decisions of the backward kernels made visible (same
 * passages as fa_fwd_debug_visits: causal block skipping, FlashAttention-2
 * review, "Proposed method"; block-sparse skipping, Stanford FlashAttention
 * summary). It writes visited_kv, uint8 [B][H][ceil(N/bn1)][ceil(N/bm1)] (pass 1
 * tile sizes, key tile major) from the dK/dV kernel and visited_q, uint8
 * [B][H][ceil(N/bm2)][ceil(N/bn2)] (pass 2 tile sizes) from the dQ kernel.
 * The caller zeroes both maps. */
int fa_bwd_debug_visits(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dO, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d, int causal, float scale,
                        const uint8_t* block_mask,
                        void* workspace, size_t workspace_bytes,
                        uint8_t* visited_kv, uint8_t* visited_q, void* stream);

/* Measurement utility, which no passage of the pages defines: the fp32
 * atomic-add rate of the accumulation a dQ-by-atomics backward would make
 * (the alternative to a separate dQ pass that the FlashAttention-2 review,
 * "Proposed method", leaves open). Enqueues one kernel of `workgroups`
 * workgroups of 256 threads; each adds 1.0f, 16 * 256 * reps times, into
 * the 32 x 32 MFMA result layout of a [64][128] fp32 block of dst (16-byte
 * aligned, dst_floats >= 8192 floats, contents overwritten by sums).
 * Adds = workgroups * 256 * 16 * reps; time it on the stream. */
int fa_atomic_add_probe(float* dst, size_t dst_floats, int workgroups, int reps, void* stream);

/* Identity of the sources this library was built from: the first 16 hex
 * digits of a SHA-256 over the kernel sources, the headers and the build
 * script, fixed at build time (static string, never NULL). A utility of
 * this library, which no passage of the pages defines: the Python binding
 * recomputes it from the sources beside the library and refuses to load a
 * library built from other sources. */
const char* fa_build_id(void);

/* Human-readable name of a status code (static string, never NULL). A
 * utility of this library: no passage of the pages defines it. */
const char* fa_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
