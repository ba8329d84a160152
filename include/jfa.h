/*
 * jfa.h -- C ABI of the jagged FlashAttention library for AMD Instinct MI355X
 * (gfx950).
 *
 * What it computes. Exact softmax attention run directly on packed ("jagged")
 * Q/K/V tensors whose sequence boundaries are given by an int32 offsets array,
 * with no padded token ("Meta's TLX Jagged Flash Attention Beats FA4 on
 * Blackwell With 3x Less Code" (ainewsbites.com), section "Why attention in GEM
 * needed a rewrite"; "Meta's 3.2K-line Triton kernel outruns FlashAttention-4
 * on jagged Blackwell attention" (theclarity.today), third paragraph).
 * In broadcast-Q mode one dense Q is shared by every sequence and its gradient
 * is summed over the whole batch (theclarity.today, second paragraph).
 * For sequence b, query row i and a visible key j:
 *     s_ij = scale * <q_i, k_j>,  LSE_i = ln sum_j exp(s_ij),
 *     O_i  = sum_j exp(s_ij - LSE_i) v_j.
 * Visible keys: every key of the row's own sequence; with causal=1 only keys
 * j <= i (local indices); with a sliding window only keys
 * i - window_left <= j <= i + window_right (the pages name sliding-window
 * attention among the variants the kernel serves, theclarity.today fourth
 * paragraph and ainewsbites.com section "Why attention in GEM needed a
 * rewrite", without defining it: this band is the usual meaning; causal is
 * the band with no left bound and right bound 0); with a block mask only keys
 * whose 128-key block is kept for the row's 128-row Q tile ("TLX porta
 * l'attenzione jagged su Blackwell" (ai-radar.it), section "The turning
 * point").
 *
 * Layouts (all row-major, contiguous):
 *   q        bf16 [lq, H, D] when broadcast_q, else [T_q, H, D]
 *   k, v     bf16 [T_k, H, D],   T_k = kv_offsets[B]
 *   o, dO    bf16 [T_q, H, D],   T_q = B*lq (row b*lq+i) when broadcast_q,
 *                                else q_offsets[B]
 *   lse      fp32 [H, T_q]       natural log of the scaled scores; -inf for a
 *                                row with no visible key (its O row is 0)
 *   delta    fp32 [H, T_q]       rowsum(dO * O)
 *   dq       bf16, shape of q;   dq_accum fp32, shape of q (the fp32 sum the
 *                                bf16 dq is rounded from)
 *   dk, dv   bf16 [T_k, H, D]
 *   offsets  int32 [B+1], offsets[0] = 0, non-decreasing
 *   mask     uint8 [B, mask_q_blocks, mask_kv_blocks], nonzero = kept
 * Device tensors must be 16-byte aligned. H*D*2 bytes is the row stride.
 *
 * Conventions for every function:
 *   - returns JFA_OK (0) or a negative JFA_ERR_* status; never throws, never
 *     aborts, never allocates device memory and never synchronises;
 *   - GPU work is enqueued on the caller's stream (a hipStream_t passed as
 *     void*; NULL is the default stream);
 *   - the caller owns every buffer; host pointers (h_*) are read during the
 *     call only; device pointers (d_* and tensors) must stay valid until the
 *     enqueued work completes;
 *   - arguments are validated on the host before anything is launched; a bad
 *     argument returns an error and launches nothing.
 */
#ifndef JFA_H
#define JFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JFA_ABI_VERSION 10

/* status codes */
#define JFA_OK                 0
#define JFA_ERR_INVALID_ARG   -1  /* null/misaligned pointer, bad size or flag */
#define JFA_ERR_BAD_OFFSETS   -2  /* offsets[0] != 0, decreasing, or overflow   */
#define JFA_ERR_UNSUPPORTED   -3  /* head_dim not 64/128, num_heads > 32768,
                                     causal or window with broadcast Q or with
                                     unequal Q/KV lengths, mask with causal or
                                     window                                   */
#define JFA_ERR_PLAN_MISMATCH -4  /* plan built for another pass/problem      */
#define JFA_ERR_WORKSPACE     -5  /* workspace too small                       */
#define JFA_ERR_HIP           -6  /* a HIP call failed: see jfa_last_hip_error */
#define JFA_ERR_BAD_MASK      -7  /* block mask missing or too small           */

/* planner passes */
#define JFA_PASS_FWD 0
#define JFA_PASS_BWD 1
#define JFA_PASS_DQ 2   /* Q-stationary dQ pass of the backward */
/* OR'ed into a FWD pass: a plan for dynamic tile fetch (see the planner) */
#define JFA_PLAN_DYNAMIC 16
/* OR'ed into any pass (not with JFA_PLAN_DYNAMIC): the unsorted ablation
   plan, tiles in enumeration order dealt round-robin (see the planner) */
#define JFA_PLAN_NATURAL 32

/* Problem description shared by the planner, jfa_fwd and jfa_bwd. */
typedef struct jfa_problem {
    int32_t batch;          /* B >= 0 sequences                                */
    int32_t num_heads;      /* 1 <= H <= 32768 (a token row of H*D bf16 stays
                               below 2^24 bytes: the kernels address a block's
                               rows with 24-bit multiples of it)               */
    int32_t head_dim;       /* D, 64 or 128                                    */
    int32_t broadcast_q;    /* 1: one dense Q [lq,H,D] shared by all sequences */
    int32_t lq;             /* rows of the shared Q (broadcast_q only), >= 0   */
    int32_t causal;         /* 1: key j visible to row i iff j <= i; needs
                               per-sequence Q with the same lengths as KV      */
    int32_t mask_q_blocks;  /* block-sparse mask dims; both 0 = dense          */
    int32_t mask_kv_blocks;
    float   softmax_scale;  /* finite and > 0; usually 1/sqrt(D)               */
    int32_t window_left;    /* sliding window: key j visible to row i only if
                               j >= i - window_left; -1 = no bound             */
    int32_t window_right;   /* ... and only if j <= i + window_right; -1 = no
                               bound (causal=1 makes it 0). Either bound needs
                               per-sequence Q with the same lengths as KV      */
} jfa_problem;

/* Sizes of a plan, filled by jfa_plan_query / jfa_plan_build. */
typedef struct jfa_plan_info {
    int32_t pass;           /* JFA_PASS_FWD, JFA_PASS_BWD or JFA_PASS_DQ, with
                               JFA_PLAN_DYNAMIC for a dynamic FWD plan         */
    int32_t num_workers;    /* W persistent workgroups the plan is dealt to
                               (DQ with broadcast Q: max(requested, G))       */
    int32_t num_tiles;      /* N tiles                                         */
    int32_t block_m;        /* rows of a Q tile (fwd) / Q block (bwd)          */
    int32_t block_n;        /* keys of a KV block (fwd) / KV tile (bwd)        */
    int32_t total_q;        /* T_q                                             */
    int32_t total_kv;       /* T_k                                             */
    int32_t sparse_rows;    /* rows of the block-sparse CSR (fwd) / columns of
                               the CSC (bwd); 0 when dense                     */
    int32_t sparse_nnz;     /* entries of its index array                      */
    int32_t max_work;       /* largest tile work                               */
    int64_t total_work;     /* sum of tile work                                */
} jfa_plan_info;

int32_t jfa_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* jfa_status_string(int32_t status);

/* The hipError_t of the last failed HIP call made by this thread. */
int32_t jfa_last_hip_error(void);

/* Compute units of HIP device `device` (the natural worker count unit). */
int32_t jfa_device_workers(int32_t device, int32_t* num_cus);

/* offsets[0] = 0, offsets[b+1] = offsets[b] + lengths[b]. h_offsets has B+1
 * entries. Lengths must be >= 0 and the total must fit int32. */
int32_t jfa_offsets_from_lengths(const int32_t* h_lengths, int32_t batch, int32_t* h_offsets);

/*
 * Host tile planner ("Meta's TLX Jagged Flash Attention Beats FA4 on
 * Blackwell" (ainewsbites.com), section "Optimizations layered on top": tiles
 * sorted on the host by KV workload, largest first, dealt to the processors
 * in a zigzag pattern; software load balancing across length skew).
 *
 * Tiles are enumerated in (b, h, t) order. FWD: t is a Q tile of block_m=256
 * rows, work = KV blocks of block_n=64 keys visited (dense: ceil(Lk/64);
 * causal: ceil(min(256(t+1), L)/64); band (window, causal): the blocks from
 * jmin/64 to jmax/64 with jmin = max(0, 256t - left), jmax = min(L - 1,
 * 256t + 255 + right) (rows past L excluded), 0 if jmax < jmin; block-sparse:
 * the 64-key blocks of the
 * 128-key mask blocks inside the sequence kept by either of the tile's two
 * 128-row mask rows). BWD: t is a KV tile of block_n=256 keys, work = Q
 * blocks of block_m=32 rows visited (dense: ceil(Lq/32); causal:
 * ceil(L/32) - 8t; block-sparse: the 32-row blocks of the 128-row mask rows
 * kept by either of the tile's two 128-key mask columns inside the
 * sequence). Tiles are stably sorted by work, descending, and sorted tile i goes
 * to worker i mod W when floor(i/W) is even, else to W-1-(i mod W).
 * DQ: the FWD tiles and work. With per-sequence Q the deal is the FWD deal.
 * With broadcast Q (every tile (b, h, t) adds into the same dQ rows of head
 * h), the G = H * ceil(lq/256) groups g = h * ceil(lq/256) + t get disjoint
 * worker ranges [g W'/G, (g+1) W'/G) of W' = max(G, min(W, G n)) workers (n the
 * largest number of chunks, below, of any group; W' = W when G = 0), and each
 * group's tiles are sorted and snake-dealt over its own range, so that every
 * worker sums one group only (one partial per worker). Since those partials
 * are summed anyway, a broadcast-Q DQ tile of more than 16 blocks is first
 * split into n = ceil(work/16) chunks of consecutive positions of its block
 * list (the first work mod n of them one block longer), listed in (b, h, t,
 * chunk) order; a chunk starting at position k0 is stored as
 * (b, h, t + ceil(lq/256) * k0, its length).
 *
 * JFA_PASS_FWD | JFA_PLAN_DYNAMIC: the same FWD tiles for dynamic fetch (the
 * role the pages give the hardware's cluster launch control next to the host
 * sort: a running workgroup claims the next tile when it needs one; bites,
 * sections "What TLX changes" and "Optimizations layered on top"). h_tiles
 * holds the whole stably sorted list (largest work first) and
 * h_worker_ptr[w] = min(w, N): worker w starts with sorted tile w, and later
 * tiles W, W+1, ... go, one at a time and in order, to whichever worker asks
 * first (a device counter, see jfa_fwd). Only the forward has this mode.
 *
 * pass | JFA_PLAN_NATURAL: the baseline the sort and zigzag deal are measured
 * against (the pages credit them with about a fifth of the forward's speed;
 * bites, "Optimizations layered on top"): no sort, tiles in enumeration
 * order (b, h, t) dealt round-robin, enumerated tile i to worker i mod W
 * (broadcast-Q DQ: within each group's workers, the groups and chunks as
 * above). info->pass does not record the flag: the plan has the layout of a
 * static plan of its pass and is used like one.
 *
 * h_q_offsets: int32 [B+1], NULL in broadcast mode. h_kv_offsets: int32 [B+1].
 * h_block_mask: NULL when mask_q_blocks = mask_kv_blocks = 0.
 * jfa_plan_query fills *info only (sizes). jfa_plan_build also writes
 *   h_worker_ptr  int32 [W+1]      tiles of worker w are [ptr[w], ptr[w+1])
 *   h_tiles       int32 [N*4]      (b, h, t, work) per tile
 *   h_sparse_ptr  int32 [sparse_rows+1], h_sparse_idx int32 [sparse_nnz]
 *                 (block-sparse only, else may be NULL): FWD and DQ = CSR
 *                 over Q tiles b*ceil(mask_q_blocks/2)+t of the 128-key
 *                 blocks c inside the sequence kept by a mask row of the
 *                 tile, stored as 4c + bits (bit k: row 2t+k keeps c; rows
 *                 past the mask or the sequence keep nothing); BWD = CSC
 *                 over KV tiles b*ceil(mask_kv_blocks/2)+t of the 128-row
 *                 mask rows m inside the sequence kept by a mask column of
 *                 the tile, stored as 4m + bits (bit k: column 2t+k keeps
 *                 m); ascending.
 * The caller copies these arrays to the device for jfa_fwd / jfa_bwd.
 */
int32_t jfa_plan_query(const jfa_problem* prob, const int32_t* h_q_offsets,
                       const int32_t* h_kv_offsets, const uint8_t* h_block_mask,
                       int32_t pass, int32_t num_workers, jfa_plan_info* info);
int32_t jfa_plan_build(const jfa_problem* prob, const int32_t* h_q_offsets,
                       const int32_t* h_kv_offsets, const uint8_t* h_block_mask,
                       int32_t pass, int32_t num_workers, jfa_plan_info* info,
                       int32_t* h_worker_ptr, int32_t* h_tiles,
                       int32_t* h_sparse_ptr, int32_t* h_sparse_idx);

/* Bytes of device scratch jfa_fwd needs for this FWD plan: 256 for a
 * dynamic plan (the tile counter), else 0. */
int32_t jfa_fwd_workspace_bytes(const jfa_problem* prob, const jfa_plan_info* info,
                                int64_t* bytes);

/*
 * Forward pass: O and LSE. One persistent launch of info->num_workers
 * workgroups walking a FWD plan (d_worker_ptr, d_tiles and, for a block mask,
 * d_sparse_ptr/d_sparse_idx, all device copies of jfa_plan_build's output).
 * d_q_offsets is NULL in broadcast mode. Every O/LSE row is written.
 * workspace: jfa_fwd_workspace_bytes bytes, 16-byte aligned (may be NULL when
 * that is 0). For a dynamic plan it holds the tile counter: it must be all
 * zero before the first launch that uses it (e.g. allocated zeroed), every
 * launch leaves it zero again, and launches that share one workspace must
 * not overlap in time (same stream, or ordered by events).
 */
int32_t jfa_fwd(const jfa_problem* prob, const jfa_plan_info* info,
                const int32_t* d_worker_ptr, const int32_t* d_tiles,
                const int32_t* d_sparse_ptr, const int32_t* d_sparse_idx,
                const int32_t* d_q_offsets, const int32_t* d_kv_offsets,
                const void* q, const void* k, const void* v,
                void* o, float* lse, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * MXFP8 variant ("TLX porta l'attenzione jagged su Blackwell" (ai-radar.it),
 * section "The turning point": products in microscaling precision, P
 * quantised to FP8 on the fly). Format: OCP MXFP8 -- E4M3 element codes
 * (uint8) sharing one E8M0 scale code c (value 2^(c-127), uint8) per block of
 * 32 elements along the contraction dimension of each product: d for Q and
 * K, 32 consecutive keys of one sequence for V (a sequence's last block may
 * be shorter; blocks never span two sequences). A block's exponent is
 * floor(log2(max |x|)) - 8 (clamped to [-127, 127]; 0 blocks: -127); its
 * elements are x / 2^e rounded to nearest even, magnitudes above 448
 * clamped. Layouts: Q codes [q rows, H, D] with scales [H, q rows, D/32]
 * (q rows = lq when broadcast, else T_q); K codes [T_k, H, D] with scales
 * [H, T_k, D/32]; V codes [T_k, H, D] with scales [H, NB, D], the blocks of
 * sequence b starting at block_offsets[b] and NB = block_offsets[B]. Codes
 * are 16-byte aligned, scales 4-byte aligned; an empty array may be NULL.
 */
/* block_offsets[0] = 0, block_offsets[b+1] = block_offsets[b] + ceil(L_b/32)
 * for the lengths given by h_kv_offsets [B+1] (host arrays). */
int32_t jfa_mx_block_offsets(const int32_t* h_kv_offsets, int32_t batch, int32_t* h_block_offsets);
/* Encode a bf16 [rows, num_heads, head_dim] tensor (Q or K; head_dim a
 * multiple of 32) into codes [rows, H, D] and scales [H, rows, D/32]. */
int32_t jfa_mx_quantize_rows(const void* src, int64_t rows, int32_t num_heads, int32_t head_dim,
                             void* codes, void* scales, void* stream);
/* Encode bf16 V [T_k, H, D] into codes [T_k, H, D] and scales [H, NB, D];
 * d_kv_offsets / d_block_offsets are device copies ([B+1]). */
int32_t jfa_mx_quantize_v(const void* v, const int32_t* d_kv_offsets,
                          const int32_t* d_block_offsets, int32_t batch, int32_t num_heads,
                          int32_t head_dim, int32_t num_blocks, void* codes, void* scales,
                          void* stream);
/*
 * MXFP8 forward: O (bf16) and LSE (fp32) as jfa_fwd, from MXFP8 Q, K, V
 * (head_dim 128; same plans, modes and workspace as jfa_fwd). S = Q K^T and
 * O = P V run as block-scaled FP8 products with fp32 accumulation; the
 * softmax is fp32, and P = exp(S - running max) <= 1 is rounded to E4M3 with
 * the fixed block scale 2^-8 before O = P V (its row sum stays fp32).
 */
int32_t jfa_fwd_mx(const jfa_problem* prob, const jfa_plan_info* info,
                   const int32_t* d_worker_ptr, const int32_t* d_tiles,
                   const int32_t* d_sparse_ptr, const int32_t* d_sparse_idx,
                   const int32_t* d_q_offsets, const int32_t* d_kv_offsets,
                   const int32_t* d_block_offsets, int32_t num_blocks,
                   const void* q_codes, const void* q_scales, const void* k_codes,
                   const void* k_scales, const void* v_codes, const void* v_scales,
                   void* o, float* lse, void* workspace, int64_t workspace_bytes, void* stream);

/* A plan on the device: the sizes of jfa_plan_build's output and device
 * copies of its arrays (sparse_ptr / sparse_idx NULL when dense). The caller
 * owns everything it points to. */
typedef struct jfa_device_plan {
    const jfa_plan_info* info;
    const int32_t* worker_ptr;
    const int32_t* tiles;
    const int32_t* sparse_ptr;
    const int32_t* sparse_idx;
} jfa_device_plan;

/* Bytes of device scratch jfa_bwd needs for this DQ plan: with broadcast Q,
 * one fp32 [256][head_dim] partial per dQ worker (dq_info->num_workers of
 * them); 0 with per-sequence Q. */
int32_t jfa_bwd_workspace_bytes(const jfa_problem* prob, const jfa_plan_info* dq_info,
                                int64_t* bytes);

/*
 * Backward pass: dQ, dK, dV for the loss sum(dO * O), given the forward's O
 * and LSE. kv_plan is a BWD plan (KV tiles), dq_plan a DQ plan (Q tiles), both
 * for this problem and these offsets. Enqueues, in stream order:
 *   1. dQ: Q-stationary persistent kernel over dq_plan (the forward's tiles),
 *      dQ accumulated in registers while the K/V blocks stream past; each
 *      tile also forms delta = rowsum(dO * O) (fp32 [H, T_q]) of its rows
 *      and writes it out. With per-sequence Q each tile writes its rows of
 *      dq_accum (fp32) and dq (bf16). With broadcast Q, dQ sums over all
 *      sequences (theclarity.today, second paragraph): each dQ worker adds up
 *      its tiles, which all belong to one (head, Q tile) group, into one fp32
 *      partial in the workspace;
 *   2. dK/dV: KV-stationary persistent kernel over kv_plan (reads delta), dK
 *      and dV accumulated per KV tile in registers and written as bf16;
 *   3. dQ reduce (broadcast Q only): the partials of each group are added in
 *      worker order into dq_accum (fp32 [lq, H, D]) and dq (bf16). The result
 *      does not depend on timing; no atomics are used anywhere.
 * dq_accum and delta are outputs too. workspace: jfa_bwd_workspace_bytes
 * bytes, 16-byte aligned (may be NULL when that is 0).
 */
int32_t jfa_bwd(const jfa_problem* prob, const jfa_device_plan* kv_plan,
                const jfa_device_plan* dq_plan, const int32_t* d_q_offsets,
                const int32_t* d_kv_offsets, const void* q, const void* k, const void* v,
                const void* o, const float* lse, const void* d_o,
                void* dq, void* dk, void* dv, float* dq_accum, float* delta,
                void* workspace, int64_t workspace_bytes, void* stream);

/*
 * The same backward, one stage at a time, for callers that interleave other
 * work or time each launch: `stages` is a bitwise OR of the JFA_BWD_* flags;
 * the selected launches are enqueued in flag order. Each stage expects the
 * outputs of the stages before it to be in place (delta for DKDV, the dQ
 * partials for DQ_REDUCE). Arguments are the same as jfa_bwd and are
 * validated the same way whatever the stages.
 */
#define JFA_BWD_PREPROCESS 1   /* delta = rowsum(dO*O) alone (not in ALL: the
                                  DQ stage forms it too)                      */
#define JFA_BWD_DQ         2   /* dQ (per-sequence Q) or dQ partials
                                  (broadcast), and delta                      */
#define JFA_BWD_DKDV       4   /* dK, dV                                       */
#define JFA_BWD_DQ_REDUCE  8   /* broadcast Q: dq_accum, dq from the partials  */
#define JFA_BWD_ALL        14
/* Modifier of the broadcast-Q dQ reduction (no effect with per-sequence Q):
 * the second of the two stages the pages describe for the batch-summed dQ
 * ("Meta's TLX Jagged Flash Attention Beats FA4 on Blackwell"
 * (ainewsbites.com), section "Optimizations layered on top") done by fp32
 * atomic adds instead of a fixed-order reduce. With JFA_BWD_DQ the stage
 * first zeroes dq_accum, then each dQ worker adds its sum over its tiles into
 * dq_accum with device-scope fp32 atomic adds (no partials are written);
 * with JFA_BWD_DQ_REDUCE the stage only rounds dq_accum to dq (bf16). The sum
 * then depends on the order in which the adds land: not bitwise reproducible
 * from run to run. The workspace is still validated but not used. */
#define JFA_BWD_DQ_ATOMIC 16
int32_t jfa_bwd_stages(int32_t stages, const jfa_problem* prob, const jfa_device_plan* kv_plan,
                       const jfa_device_plan* dq_plan, const int32_t* d_q_offsets,
                       const int32_t* d_kv_offsets, const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* d_o,
                       void* dq, void* dk, void* dv, float* dq_accum, float* delta,
                       void* workspace, int64_t workspace_bytes, void* stream);

/*
 * jfa_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * same backward with the same arguments except the workspace, which is a
 * scratch area of JFA_NOALLOC_SCRATCH_BYTES inside the library itself, one
 * per GPU (each GPU the library runs on holds it until the process ends);
 * the call allocates and frees nothing. Returns JFA_ERR_WORKSPACE, before
 * anything is launched, when the DQ plan needs more than that
 * (jfa_bwd_workspace_bytes: with a broadcast Q, 256 * head_dim * 4 bytes per
 * dQ worker, i.e. at most 256 dQ workers at head_dim 128 and 512 at 64;
 * per-sequence Q needs none). Nothing in the area has to start at zero: every
 * dQ worker writes its whole partial before the reduce reads it. Every call
 * on one GPU uses the same area, which keeps the last call's contents: two
 * calls whose work overlaps in time on one GPU (streams not ordered by
 * events) race on it, so order them.
 */
#define JFA_NOALLOC_SCRATCH_BYTES (32 << 20)
int32_t jfa_bwd_noalloc(const jfa_problem* prob, const jfa_device_plan* kv_plan,
                        const jfa_device_plan* dq_plan, const int32_t* d_q_offsets,
                        const int32_t* d_kv_offsets, const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* d_o,
                        void* dq, void* dk, void* dv, float* dq_accum, float* delta, void* stream);

/*
 * MXFP8 dQ pass ("TLX porta l'attenzione jagged su Blackwell" (ai-radar.it),
 * section "The turning point": the MXFP8 version of the kernel; its backward,
 * here the dQ pass): the JFA_BWD_DQ stage with its three products as
 * block-scaled FP8 MFMAs (head_dim 128):
 *   S  = Q K^T    Q and K encoded along d (the MXFP8 forward's encodings),
 *   dP = dO V^T   dO and V encoded along d (jfa_mx_quantize_rows),
 *   dQ += dS K    K encoded along the keys of its sequence in 32-key blocks
 *                 (jfa_mx_quantize_v applied to K), and dS = P (dP - delta)
 *                 rounded to E4M3 on the fly with one E8M0 scale per (query
 *                 row, 32-key block): the smallest power of two 2^e with
 *                 max|dS| / 2^e <= 448, so no value is clamped (a block below
 *                 2^-100 is sent as zeros).
 * P = exp(S - LSE) and dS are fp32; delta = rowsum(dO * O) is formed from the
 * bf16 dO and O and written out, as by JFA_BWD_DQ. Outputs as JFA_BWD_DQ:
 * per-sequence Q: dq and dq_accum; broadcast Q: the per-worker partials in
 * the workspace (same size as jfa_bwd's), which jfa_bwd_stages with
 * JFA_BWD_DQ_REDUCE turns into dq_accum and dq. The dK/dV pass comes after
 * this call, which writes the delta it needs: bf16 (jfa_bwd_stages with
 * JFA_BWD_DKDV) or MXFP8 (jfa_bwd_dkdv_mx).
 * Layouts: codes [rows, H, D] and scales [H, rows, D/32] for the operands
 * encoded along d (rows: lq or T_q for Q, T_k for K and V, T_q for dO); K
 * along keys: codes [T_k, H, D], scales [H, NB, D] with the blocks of
 * sequence b starting at d_key_block_offsets[b] (device copy of
 * jfa_mx_block_offsets' output, NB = num_key_blocks). Scale arrays 4-byte
 * aligned, codes 16-byte aligned (either may be NULL when it is empty); the
 * caller owns everything.
 */
typedef struct jfa_mx_bwd_operands {
    const void* q_codes;
    const void* q_scales;
    const void* k_codes;
    const void* k_scales;
    const void* v_codes;
    const void* v_scales;
    const void* do_codes;
    const void* do_scales;
    const void* kk_codes;     /* K along keys */
    const void* kk_scales;
} jfa_mx_bwd_operands;
int32_t jfa_bwd_dq_mx(const jfa_problem* prob, const jfa_device_plan* dq_plan,
                      const int32_t* d_q_offsets, const int32_t* d_kv_offsets,
                      const int32_t* d_key_block_offsets, int32_t num_key_blocks,
                      const void* o, const float* lse, const void* d_o,
                      const jfa_mx_bwd_operands* ops, void* dq, float* dq_accum, float* delta,
                      void* workspace, int64_t workspace_bytes, void* stream);

/*
 * MXFP8 dK/dV pass ("TLX porta l'attenzione jagged su Blackwell" (ai-radar.it),
 * section "The turning point": the MXFP8 version of the kernel; its backward,
 * here the dK/dV pass): the JFA_BWD_DKDV stage with its four products as
 * block-scaled FP8 MFMAs (head_dim 128):
 *   S  = Q K^T    Q and K encoded along d (the MXFP8 forward's encodings),
 *   dP = dO V^T   dO and V encoded along d (jfa_mx_quantize_rows),
 *   dV = P^T dO   dO encoded along its rows in 32-row blocks of one sequence
 *                 (jfa_mx_quantize_v applied to dO with the row offsets of
 *                 the sequences: b*lq with a broadcast Q, else q_offsets);
 *                 P = exp(S - LSE) <= 1 rounded to E4M3 on the fly with the
 *                 fixed block scale 2^-8,
 *   dK = scale dS^T Q   Q encoded along its rows (jfa_mx_quantize_v applied
 *                 to Q with offsets [0, lq] for a broadcast Q, else
 *                 q_offsets); dS = P (dP - delta) rounded to E4M3 on the fly
 *                 with one E8M0 scale per (key, 32-row block): the smallest
 *                 power of two 2^e with max|dS| / 2^e <= 448, so nothing is
 *                 clamped (a block below 2^-100 is sent as zeros).
 * P, dS and the dK/dV accumulators are fp32; dk and dv are written as bf16
 * [T_k, H, D]. lse is the forward's, delta = rowsum(dO * O) (written by the
 * dQ pass, bf16 or MXFP8, or by JFA_BWD_PREPROCESS). kv_plan is a BWD plan.
 * Along-rows layouts: codes [rows, H, D], scales [H, NB, D] with the blocks
 * of sequence b starting at d_*_row_block_offsets[b] (device copies of
 * jfa_mx_block_offsets' output for those row offsets; the Q one is not read
 * with a broadcast Q, whose blocks are those of its lq rows). Scale arrays
 * 4-byte aligned, codes 16-byte aligned (either may be NULL when empty); the
 * caller owns everything.
 */
typedef struct jfa_mx_dkdv_operands {
    const void* q_codes;      /* Q along d */
    const void* q_scales;
    const void* k_codes;      /* K along d */
    const void* k_scales;
    const void* v_codes;      /* V along d */
    const void* v_scales;
    const void* do_codes;     /* dO along d */
    const void* do_scales;
    const void* qr_codes;     /* Q along its rows */
    const void* qr_scales;
    const void* dor_codes;    /* dO along its rows */
    const void* dor_scales;
} jfa_mx_dkdv_operands;
int32_t jfa_bwd_dkdv_mx(const jfa_problem* prob, const jfa_device_plan* kv_plan,
                        const int32_t* d_q_offsets, const int32_t* d_kv_offsets,
                        const int32_t* d_q_row_block_offsets, int32_t num_q_row_blocks,
                        const int32_t* d_do_row_block_offsets, int32_t num_do_row_blocks,
                        const float* lse, const float* delta, const jfa_mx_dkdv_operands* ops,
                        void* dk, void* dv, void* stream);

/*
 * Executed-tile log, for checking the kernels' walk over their plans (debug
 * builds of the library only, libjfa_debug.so; the product library returns
 * JFA_ERR_UNSUPPORTED and logs nothing). While set, every launch of the bf16
 * forward, dK/dV and dQ kernels (jfa_fwd, jfa_bwd, jfa_bwd_stages,
 * jfa_bwd_noalloc) has each worker record, in the order it takes them, the
 * tiles it executes: worker w's area starts at int32 index
 * w * (8 + 8 * records_per_worker) of d_log; area[0] = the number of tiles
 * the worker took, and tile n (n < records_per_worker) is the 8 int32 at
 * area + 8 + 8 n:
 *   {pass (0 forward, 1 dK/dV, 2 dQ), worker, b, h, t, work, blocks, flags}
 * with (b, h, t, work) the plan's record (the dQ pass's t as in its plan),
 * blocks = the worker's blocks streamed so far at the tile's end (-1 for the
 * forward, which logs a tile when its loader takes it) and flags the
 * indices checked against the problem: 1 b outside the batch, 2 h outside
 * the heads, 4 t outside the sequence's tiles. d_log: device memory, 16-byte
 * aligned, of at least num_workers * (8 + 8 * records_per_worker) int32 for
 * every launch made while it is set, owned by the caller, who zeroes the
 * area before a launch whose log it reads (each launch writes over the
 * last); launches that log must not overlap in time. NULL turns the log
 * off. The setting is process-wide. The debug build waits for its log
 * stores after each record, so it runs slower than the product library.
 */
int32_t jfa_debug_tile_log(int32_t* d_log, int32_t records_per_worker);

#ifdef __cplusplus
}
#endif

#endif /* JFA_H */
