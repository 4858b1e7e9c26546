/*
 * paged_attn.h — C ABI of the MI355X (gfx950) paged-KV attention forward library.
 *
 * One call computes, for every query token of a packed varlen batch and every
 * query head, O = softmax(scale * Q K^T + mask) V over that sequence's keys,
 * which live in a paged KV cache, plus LSE = ln sum exp(scale * Q K^T) over the
 * visible keys.  The operation and its pieces are the ones described on the
 * pages about paged attention:
 *
 *  - "Triton-TLE rewrite of Tencent HPC-Ops Attention" (flagos.csdn.net),
 *    §1.2: dynamic decode in three stages — Assign (cut each KV sequence into
 *    tiles and build a load-balanced task map), Split-K compute (a persistent
 *    grid walks the task map and emits a partial output and LSE per KV chunk)
 *    and Combine (LSE-weighted merge, equal to full attention); prefill with
 *    QK, causal mask, fp32 online softmax, PV and a normalising epilogue;
 *    block table lookup of physical pages; 128x128 block-mask tile skipping;
 *    FP8 (e4m3) K/V with quantisation scales.  §3.2: NHD and HND caches
 *    differ only in strides over logical (page, slot, head, dim) coordinates.
 *  - "Chunked Prefill kernel optimisation: Triton hybrid attention" (xdnf.cn):
 *    a chunk of prefill tokens and many decode rows in one launch; decode rows
 *    see their whole history, a chunk is causal within itself.
 *  - "HiLS-Attention sliding-window forward" (flagos.csdn.net), §3: LSE in
 *    natural log, output layout (B, Hq, Lq, Dv) through strides, sliding
 *    window with expand_to_chunk and landmark masking (j + 1) mod C != 0,
 *    split-KV decode.
 *  - "vLLM Triton Attention Backend Deep Dive" (papercache), §3: Q blocks
 *    group all query heads of one KV head; a persistent grid of fixed size
 *    reads its work from GPU metadata (so a launch is graph-capturable).
 *
 * Conventions for every entry point
 *  - Every function returns a pa_status; PA_OK is 0.
 *  - Device pointers are HIP device memory of the current device; host
 *    pointers are named *_h.  The library allocates no memory, never
 *    synchronises, never reads device memory on the host and keeps no pointer
 *    after a call returns.  The caller owns every buffer, the workspace
 *    included.  All argument checks run before the first launch: a call that
 *    fails a check has no side effects; a HIP runtime failure (PA_ERR_HIP)
 *    may leave the launches issued before it enqueued.
 *  - Calls are re-entrant; two calls that share a workspace must be ordered
 *    on one stream.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,   /* null pointer, inconsistent shape/stride, bad size */
  PA_ERR_UNSUPPORTED = 2,   /* dtype mix, head_dim, GQA ratio or layout not built */
  PA_ERR_WORKSPACE = 3,     /* workspace null, misaligned or too small */
  PA_ERR_HIP = 4,           /* a HIP runtime call failed; see paged_attn_last_hip_error */
  PA_ERR_SCRATCH = 5        /* paged_attn_fwd_noalloc: the call needs more workspace than
                               PA_NOALLOC_SCRATCH_BYTES */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_BF16 = 1,
  PA_F8E4M3 = 2,            /* OCP E4M3FN */
  PA_U8 = 3
} pa_dtype;

/* A strided view of device memory.  shape/stride are in elements; unused
 * trailing entries are ignored.  The innermost (last) dimension must have
 * stride 1 except where noted. */
typedef struct pa_tensor {
  void* data;
  int32_t dtype;            /* pa_dtype */
  int32_t rank;
  int64_t shape[4];
  int64_t stride[4];
} pa_tensor;

typedef enum pa_scale_mode {
  PA_SCALE_NONE = 0,
  PA_SCALE_PER_TENSOR = 1,      /* q_scale, k_scale, v_scale: one fp32 each */
  PA_SCALE_PER_PAGE_HEAD = 2,   /* q_scale: one fp32; k_scale, v_scale: fp32 [num_pages, Hkv] */
  /* A flag OR'd into either mode above: q_scale is fp32 [total_q, Hq],
   * contiguous, one scale per (query token, query head) — the FP8 decode
   * quantisation of "Triton-TLE rewrite of Tencent HPC-Ops Attention", §3
   * Dynamic Decode (Q per token and head, K/V per tensor). */
  PA_SCALE_Q_PER_TOKEN_HEAD = 4
} pa_scale_mode;

/* FP8 dequantisation scales (device pointers, so a call never reads them on
 * the host and stays capturable in a HIP graph).  Value = e4m3(x) * scale;
 * every scale must be finite and > 0.  mode = PA_SCALE_PER_TENSOR or
 * PA_SCALE_PER_PAGE_HEAD, optionally | PA_SCALE_Q_PER_TOKEN_HEAD; any other
 * value is PA_ERR_INVALID_ARG.
 * Required when Q/K/V are PA_F8E4M3, ignored otherwise. */
typedef struct pa_scales {
  int32_t mode;             /* pa_scale_mode */
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
} pa_scales;

typedef struct pa_params {
  /* sizes; each must agree with the tensors passed to paged_attn_fwd */
  int32_t num_seqs;             /* B */
  int32_t num_q_heads;          /* Hq */
  int32_t num_kv_heads;         /* Hkv; Hq % Hkv == 0 and 128 % (Hq / Hkv) == 0 */
  int32_t head_dim;             /* 64 or 128 */
  int32_t page_size;            /* a power of two */
  int32_t num_pages;            /* physical pages in the cache */
  int32_t max_pages_per_seq;    /* columns of block_table */
  int32_t block_table_stride;   /* elements between rows of block_table (>= max_pages_per_seq) */
  int32_t total_q;              /* query tokens = query_start_loc[B] */
  /* scores and masking */
  float softmax_scale;          /* multiplies Q.K (fp32, used as given); finite and > 0 */
  int32_t causal;               /* 1: key j visible only if j <= pos (bottom-right aligned) */
  int32_t window;               /* > 0: sliding window of this many keys ending at pos */
  int32_t window_expand_to_chunk; /* 1: window start rounded down to a multiple of landmark_chunk */
  int32_t landmark_chunk;       /* C > 0: hide keys with (j + 1) % C == 0 */
  int32_t block_mask_tile;      /* tile edge of block_mask in tokens; multiple of 64; 0 = 128 */
  /* scheduling */
  int32_t num_workers;          /* P persistent workgroups; 0 = two per compute unit */
  int32_t split_min_units;      /* L_min: fewest 64-key units a worker is given; 0 = 8 */
  int32_t force_split_units;    /* > 0: every worker gets exactly this many units (testing) */
  int32_t max_partial_slots;    /* capacity for split partial outputs; 0 = 2 * P (2 * (P + 1) for an odd P) */
  int32_t flags;                /* reserved, must be 0 */
  int32_t split_mode;           /* pa_split_mode */
  int32_t static_splits;        /* PA_SPLIT_STATIC: S >= 1 splits per Q-block */
  int32_t max_q_len;            /* 0, or a bound on every sequence's q_len known to the caller
                                   (a scheduler's max query length).  When max_q_len * Hq / Hkv
                                   <= 16 every Q-block is small and a kernel built without the
                                   prefill path runs (faster decode).  A sequence longer than
                                   the bound is device error PA_DEV_QLEN_HINT (outputs then
                                   unspecified). */
  int32_t min_q_len;            /* 0, or a bound below every non-zero q_len (a scheduler's
                                   prefill chunk size).  When min_q_len * Hq / Hkv > 16 every
                                   Q-block is large and a kernel built without the decode path
                                   runs (faster prefill).  A shorter non-empty sequence is
                                   device error PA_DEV_QLEN_HINT.  Must not exceed max_q_len
                                   when both are set. */
  int32_t pair_weight;          /* 1..99: percent of each worker pair's 2L units given to its
                                   first worker (the workgroup dispatched first onto a compute
                                   unit, which the hardware favours); 50 is the even split.
                                   0 = PA_PAIR_WEIGHT_SMALL with the small-Q-block kernel,
                                   PA_PAIR_WEIGHT_GENERAL otherwise (measured on MI355X) */
  int32_t fused_combine;        /* 0: a Combine kernel of its own after the attention kernel;
                                   1: fused Combine — the workgroup that finishes a split
                                   Q-block's last piece merges its partials (a per-Q-block
                                   counter in the workspace, partials through device-coherent
                                   accesses), one launch fewer.  Measured slower on MI355X
                                   (the merges land on the kernel's tail), so not the default */
  int32_t qblock_per_kv_head;   /* 0: the library's choice: a decode-only dynamic call (max_q_len
                                   set, max_q_len * Hq / Hkv <= 16) with Hkv % 4 == 0 and
                                   max_q_len * (Hq / Hkv) * (Hkv / 4) <= 16, and no block mask, gets
                                   one Q-block per sequence holding all its query heads, whose units
                                   are (64-key tile, kv head) pairs with the kv head fastest: the
                                   four waves of a workgroup then read the same keys of different
                                   kv heads together, which an NHD cache (kv heads adjacent in a
                                   page) serves at a higher rate.  1: always one Q-block per kv
                                   head. */
} pa_params;

#define PA_PAIR_WEIGHT_SMALL 60
#define PA_PAIR_WEIGHT_GENERAL 50

/* How the keys of each Q-block are cut into splits.
 *  PA_SPLIT_DYNAMIC  Assign builds a balanced task map on the device from the
 *                    real sequence lengths ("Triton-TLE rewrite of Tencent
 *                    HPC-Ops Attention", §1.2 and §3.3, dynamic Split-K).
 *  PA_SPLIT_STATIC   no task map: every Q-block (b, g) is cut into
 *                    static_splits runs of ceil(tiles / S) 64-key tiles and
 *                    workgroup i takes split i % S of Q-block i / S (the same
 *                    page's static Split-K: a fixed split count, no
 *                    rebalancing).  S = 1 is the no-split kernel: one
 *                    workgroup per Q-block writes the output, no Combine.
 *                    Requires q_len * Hq / Hkv <= 16 for every sequence
 *                    (device error PA_DEV_STATIC_ROWS otherwise, those rows
 *                    unwritten), no block mask, and, for S > 1,
 *                    B * Hkv * S <= max_partial_slots.  Two launches (one
 *                    when S = 1) after a one-thread header reset, instead of
 *                    Assign's. */
typedef enum pa_split_mode {
  PA_SPLIT_DYNAMIC = 0,
  PA_SPLIT_STATIC = 1
} pa_split_mode;

/* Where the Assign task map sits inside a workspace (byte offsets), for tests
 * that copy the workspace to the host and check the map bit for bit. */
typedef struct pa_workspace_layout {
  size_t header;          /* int32[16]: U, P, L, n_qb, n_slots, n_combine, n_workers, error, max_slots */
  size_t seq_qb_base;     /* int32[B + 1]: first Q-block of each sequence */
  size_t qb_desc;         /* int32[n_qb_max][8]: b, g, t0, nt, q0, q_len, seq_len, 0 */
  size_t unit_prefix;     /* int32[n_qb_max + 1] */
  size_t n_splits;        /* int32[n_qb_max] */
  size_t slot_base;       /* int32[n_qb_max], -1 when not split */
  size_t combine_list;    /* int32[n_qb_max] */
  size_t done;            /* int32[n_qb_max]: finished pieces per split Q-block (fused Combine) */
  size_t partial_lse;     /* float[max_slots][slot_rows] */
  size_t partial_o;       /* float[max_slots][slot_rows][head_dim] */
  size_t total;           /* bytes needed */
  int32_t n_qb_max;
  int32_t max_slots;
  int32_t num_workers;
  int32_t slot_rows;      /* rows per partial slot: 16 when every Q-block is known to be small
                             (PA_SPLIT_STATIC, or max_q_len * Hq / Hkv <= 16), max_q_len * Hq with
                             sequence Q-blocks, else 128 */
  int32_t qblock_heads;   /* query heads per token in a Q-block's rows: Hq for sequence Q-blocks
                             (see pa_params.qblock_per_kv_head), else Hq / Hkv */
} pa_workspace_layout;

typedef struct pa_device_info {
  int32_t compute_units;
  int32_t lds_bytes_per_workgroup;
  int32_t default_workers;
  char arch[64];
} pa_device_info;

/* Error word values written by the device into header[7]. */
typedef enum pa_device_error {
  PA_DEV_OK = 0,
  PA_DEV_BAD_QSL = 1,        /* query_start_loc not a non-decreasing prefix ending at total_q */
  PA_DEV_BAD_QLEN = 2,       /* some q_len > seq_len */
  PA_DEV_SLOTS = 3,          /* more split partials than max_partial_slots */
  PA_DEV_BAD_PAGE = 5,       /* a block_table entry needed for a key is outside [0, num_pages) */
  PA_DEV_STATIC_ROWS = 6,    /* PA_SPLIT_STATIC with a sequence of q_len * Hq / Hkv > 16 */
  PA_DEV_QLEN_HINT = 7       /* a q_len above params->max_q_len, or non-zero below min_q_len */
} pa_device_error;

/*
 * paged_attn_fwd — the whole forward pass, enqueued on `stream`: Assign (one
 * workgroup builds the task map in the workspace), then the persistent
 * split-K attention kernel (P workgroups), then Combine (or, with
 * fused_combine, the last workgroup on each split Q-block merges it);
 * with PA_SPLIT_STATIC a one-workgroup header reset replaces Assign.
 *
 *  q            [total_q, Hq, d], dtype f32 | bf16 | e4m3; strides for the
 *               first two dims are free (d contiguous).
 *  k_cache,     logical [num_pages, page_size, Hkv, d] (page, slot, head,
 *  v_cache      dim) with free strides on the first three dims, so an NHD
 *               cache [pages, slot, head, d] and an HND cache
 *               [pages, head, slot, d] are both passed by permuting strides.
 *               Same dtype as q.  Keys j >= seq_len of a sequence never
 *               affect a result and may hold anything (NaN included); with
 *               page_size >= 64 the rest of the 64-slot tile holding a
 *               sequence's last key is read (and discarded), so those slots
 *               must be addressable memory of the cache, as they are.
 *  block_table  int32 [B, max_pages_per_seq] (row stride
 *               params->block_table_stride); entry [b, j / page_size] is the
 *               physical page of key j of sequence b.  Entries past a
 *               sequence's last page may be read (the page-table window of a
 *               sequence covers up to 128 entries, clamped to
 *               max_pages_per_seq - 1) but never affect a result, so they
 *               may hold anything (e.g. -1).
 *  seq_lens     int32 [B]: keys of each sequence, counting its new tokens.
 *  query_start_loc int32 [B + 1]: query rows of sequence b are
 *               [qsl[b], qsl[b+1]); token i of the q_len = qsl[b+1] - qsl[b]
 *               new tokens sits at position seq_len - q_len + i.
 *  block_mask   optional (NULL = none) u8 [B, H_m, n_q_tiles, n_k_tiles],
 *               H_m in {1, Hq}, free strides; tile (pos / T, j / T) with
 *               T = block_mask_tile must be non-zero for key j to be visible.
 *               Tiles above the causal diagonal are ignored.
 *  scales       required for e4m3 inputs, else NULL.
 *  out          [total_q, Hq, d] f32 for f32 inputs, bf16 otherwise; free
 *               strides on the first two dims (e.g. (B=1, Hq, Lq, d) storage).
 *  lse          f32 [total_q, Hq], free strides: natural-log LSE.
 *               Rows with no visible key get O = 0 and LSE = -inf.
 *  workspace    device memory of at least paged_attn_workspace_size bytes,
 *               256-byte aligned; its contents need no initialisation and are
 *               overwritten (the task map stays there after the call).
 *  stream       a hipStream_t (NULL = default stream).
 */
pa_status paged_attn_fwd(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* query_start_loc, const pa_tensor* block_mask,
                         const pa_scales* scales, pa_tensor* out, pa_tensor* lse,
                         const pa_params* params, void* workspace, size_t workspace_bytes,
                         void* stream);

/* paged_attn_fwd_noalloc — paged_attn_fwd for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  The arguments and results are those of
 * paged_attn_fwd without workspace / workspace_bytes: the workspace is instead
 * a library-owned device array of PA_NOALLOC_SCRATCH_BYTES (256-byte aligned),
 * one per device, present from the library's load on that device until the
 * process ends.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks up the
 * array's address there.  A call whose paged_attn_workspace_size exceeds
 * PA_NOALLOC_SCRATCH_BYTES returns PA_ERR_SCRATCH before any launch.  On a
 * 256-CU device with the default 512 workers, d = 128 and 128-row partial
 * slots, the slots take 64.5 MiB and the rest holds the task map of about
 * 150,000 Q-blocks (n_qb_max = Hkv * (B + ceil(total_q * Hq / Hkv / 128)));
 * a small-Q-block call (16-row slots) needs about 8 MiB for its slots.
 * Every call on one device shares that
 * device's array and leaves the previous call's task map in it (each call
 * rewrites all it reads): calls that overlap in time on one device race and
 * must be ordered on one stream.  Kernel timing (paged_attn_kernel_timing)
 * records no events for this entry point. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)
pa_status paged_attn_fwd_noalloc(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* query_start_loc, const pa_tensor* block_mask,
                                 const pa_scales* scales, pa_tensor* out, pa_tensor* lse,
                                 const pa_params* params, void* stream);

/* Bytes of workspace paged_attn_fwd needs for `params` (host only; queries the
 * current device's compute-unit count when params->num_workers is 0).  The
 * caller allocates it once and passes it to every call: a closed form on the
 * host, so no call allocates or frees memory ("HiLS-Attention sliding-window
 * forward", §3 stage 3: per-call allocation and lookup made up most of a
 * wrapper's time around a short kernel).  Decode-only calls (max_q_len * G
 * <= 16, or PA_SPLIT_STATIC) need 16-row partial slots, others 128-row. */
pa_status paged_attn_workspace_size(const pa_params* params, size_t* bytes);

/* Offsets of the task map inside the workspace (host only), for tests that
 * copy the workspace to the host and compare the Assign task map ("Triton-TLE
 * rewrite of Tencent HPC-Ops Attention", §1.2 and §3.3) bit for bit with a
 * CPU specification.  It takes the place of a call that would decode the map
 * itself: the map is plain int32 arrays, so their offsets are all a reader
 * needs. */
pa_status paged_attn_workspace_layout(const pa_params* params, pa_workspace_layout* layout);

/* The split policy: picks PA_SPLIT_STATIC (and its S) or PA_SPLIT_DYNAMIC
 * for a batch from its metadata in host memory, the host-side choice of a
 * kernel variant by sequence shape that "Triton-TLE rewrite of Tencent HPC-Ops
 * Attention", §1.2 and §3 describe, with the grid-saturation test of
 * "HiLS-Attention", split-KV decode.  Static is chosen only when every
 * sequence fits one small Q-block, there is no block mask, and the static
 * cut's busiest workgroup carries no more 64-key tiles than the dynamic
 * task map's would plus the cost of its Assign launch (counted as
 * PA_POLICY_ASSIGN_UNITS tiles) and of a Combine (PA_POLICY_COMBINE_UNITS);
 * among static cuts the one with the fewest tiles on its busiest workgroup
 * wins.  Writes split_mode and static_splits; reads nothing on the device
 * except, when params->num_workers is 0, the compute-unit count. */
#define PA_POLICY_ASSIGN_UNITS 3
#define PA_POLICY_COMBINE_UNITS 2
pa_status paged_attn_plan_split(const pa_params* params, const int32_t* seq_lens_h,
                                const int32_t* query_start_loc_h, int32_t has_block_mask,
                                int32_t* split_mode, int32_t* static_splits);

/* Host-side check of batch metadata held in host memory: query_start_loc is a
 * prefix ending at total_q, 0 <= q_len <= seq_len, every block_table entry a
 * sequence needs is in [0, num_pages), and (when block_mask_h is given, a
 * dense [B, mask_heads, n_q_tiles, n_k_tiles] array, its three trailing
 * dimensions passed as mask_heads / mask_q_tiles / mask_k_tiles since a host
 * pointer carries no shape) the mask covers every sequence.  The rules are
 * those of the paged layout and varlen packing ("Triton-TLE rewrite of
 * Tencent HPC-Ops Attention", §1.2 block table, §3.2 logical page / slot
 * coordinates).  Runs no device code; paged_attn_fwd itself never reads host
 * copies and checks the same rules on the device (error word). */
pa_status paged_attn_validate_host(const pa_params* params, const int32_t* seq_lens_h,
                                   const int32_t* query_start_loc_h, const int32_t* block_table_h,
                                   const uint8_t* block_mask_h, int32_t mask_heads,
                                   int32_t mask_q_tiles, int32_t mask_k_tiles);

/* Compute units, LDS per workgroup and the default worker count of `device`:
 * the persistent grid is sized to the machine, not to the batch ("vLLM
 * Triton Attention Backend Deep Dive", §3: a fixed grid reading its work from
 * GPU metadata), two workgroups per compute unit. */
pa_status paged_attn_device_info(int32_t device, pa_device_info* info);

/* Static text for a status code. */
const char* paged_attn_status_string(pa_status status);

/* The last HIP error code seen by the calling thread (0 = none). */
int32_t paged_attn_last_hip_error(void);

/* Kernel timing for benchmarks: while enabled, every paged_attn_fwd records
 * HIP events on its own stream around each of its three launches.
 * paged_attn_kernel_timing_read waits for the recorded events, returns the
 * summed milliseconds per launch and the number of calls, and clears them. */
pa_status paged_attn_kernel_timing(int32_t enable);
pa_status paged_attn_kernel_timing_read(float* ms_assign, float* ms_attention, float* ms_combine,
                                        int32_t* calls);

#ifdef __cplusplus
}
#endif
#endif /* PAGED_ATTN_H */
