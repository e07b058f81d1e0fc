/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged decode-attention library.
 *
 * The operation (asynchronous-KV-prefetch review, sections 3.2-3.4 and 4.1;
 * PagedAttention answer, section 3): one decode step of attention for a batch
 * of sequences whose keys and values live in fixed-size blocks of a shared
 * physical pool.  For sequence b and query head h (kv head h / (Hq / Hkv)),
 * every token t < context_lens[b] sits in block block_tables[b][t / 16] at
 * slot t % 16, and
 *     out[b][h] = softmax_t(scale * q[b][h] . K_t) . V_t
 * computed with an fp32 online softmax and fp32 accumulation, rounded once to
 * fp16 (round to nearest even).
 *
 * How the blocks are walked (review, section 3.4, Algorithm 1): a work-group
 * owns a block range [s, e) of one (sequence, KV head); its w wavefronts take
 * blocks s + wave, s + wave + w, ...  Before computing block j a wavefront
 * issues the fetch of block j + w (when j + w < e) so that its memory latency
 * overlaps the compute of block j.  `pa_options.prefetch` chooses how that
 * fetch is made; results are bitwise identical in every mode.

 *
 * Ranges are split-context partitions of partition_blocks blocks, one
 * work-group each (grid: KV head x sequence x partition); when a sequence
 * has several, a second kernel merges their partial softmax states (the
 * answer's "reduce output" step).  Results are deterministic for a given
 * plan; different partition sizes or wave counts round differently (all
 * within the fp32 accumulation error).
 *
 * Conventions
 *  - Tensor pointers are DEVICE pointers, owned by the caller; the library
 *    keeps no reference after a call returns and allocates nothing.
 *  - fp16 means IEEE binary16 bits.  Layouts are row-major:
 *        q, out       [num_seqs][num_q_heads][128]
 *        k_cache      [num_blocks][num_kv_heads][16][16][8]
 *                     (dim group g, token t, dim 8g+i): the 16 bytes of one
 *                     token's dims 8g..8g+7 are one piece, and the 16 tokens'
 *                     pieces of a group are 256 contiguous bytes
 *        v_cache      [num_blocks][num_kv_heads][16][128]   (token, dim)
 *        block_tables [num_seqs][max_blocks_per_seq]  int32 physical block ids
 *        context_lens [num_seqs]                      int32 tokens to attend
 *    Each (block, kv head) slice of K and of V is one contiguous 4 KiB piece.
 *    K's grouping lets one 128-bit load per lane deliver an MFMA operand
 *    (token on the lane's column, 8 dims in the lane) while every load
 *    instruction still reads 1 KiB of contiguous memory.
 *  - All pointers must be 16-byte aligned; out must not alias an input.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Argument checks are host-only and never read device memory.
 *    Faults during execution surface at the caller's next synchronisation.
 *  - Data-dependent preconditions cannot be checked on the host:
 *        0 <= block_tables[b][j] < num_blocks   for j < ceil(ctx_b / 16)
 *        context_lens[b] <= max_blocks_per_seq * 16
 *    Violating the first is undefined behaviour unless a debug error word is
 *    given (then the kernel flags it and reads block 0 instead).  Context
 *    lengths beyond the table are clamped to it (flagged in debug mode).
 *    context_lens[b] <= 0 yields an all-zero output row.
 *  - Return values are PA_* status codes; nothing is printed, nothing aborts,
 *    no C++ exception crosses this boundary.
 *  - Calls are reentrant for distinct out / workspace / debug buffers.  Two
 *    calls that overlap in time must not share a workspace.
 *  - Workspace (when the plan has several partitions, see
 *    paged_attn_workspace_size): device memory owned by the caller, 16-byte
 *    aligned, any contents; it holds fp32 partial states between the two
 *    kernels of one call.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 8
#define PA_HEAD_DIM 128
#define PA_BLOCK_SIZE 16
#define PA_G_MAX 16      /* query heads per KV head */
#define PA_WAVES_MAX 8   /* wavefronts per work-group */

enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1, /* null pointer, bad count, misaligned pointer */
    PA_ERR_UNSUPPORTED = 2, /* head_dim != 128, block_size != 16, g > PA_G_MAX,
                               an option outside its range, or a plan whose
                               work-group needs more than the 160 KiB of LDS
                               a gfx950 work-group can hold */
    PA_ERR_WORKSPACE = 3,   /* plan needs a workspace that is missing or too small */
    PA_ERR_HIP = 4          /* a kernel launch failed (hipGetLastError) */
};

/* How block j + w is fetched while block j is computed. */
enum pa_prefetch {
    PA_PREFETCH_OFF = 0,  /* load block j, wait, compute: no look-ahead */
    PA_PREFETCH_L2 = 1,   /* touch every 128 B line of block j + k*w so it is
                             brought into L2 / Infinity Cache; data discarded */
    PA_PREFETCH_REG = 2,  /* load block j + k*w into registers (k = 1 or 2
                             buffers ahead) */
    PA_PREFETCH_BOTH = 3, /* REG for block j + w, plus an L2 touch of
                             block j + (1 + k)*w */
    PA_PREFETCH_LDS = 4   /* block j + k*w copied straight from HBM into
                             one of k+1 LDS slots of the wavefront (no
                             registers; k = 1 or 2), read out when its turn
                             comes; fused structure only */
};

/* What the caches hold. */
enum pa_kv_dtype {
    PA_KV_F16 = 0,  /* IEEE binary16 (paged_attn_decode) */
    PA_KV_E4M3 = 1  /* OCP FP8 E4M3 with per-tensor scales
                       (paged_attn_decode_fp8) */
};

/* Which sequence each row of the launch grid takes.  Work-groups start in
   grid order, so starting the longest sequences first shortens the tail of a
   ragged batch.  The result does not depend on the order. */
enum pa_seq_order {
    PA_ORDER_AUTO = 0,          /* LONGEST_FIRST when 2 <= num_seqs <=
                                   PA_RANK_MAX_SEQS and the grid has more
                                   work-groups than the CUs hold at once,
                                   else NATURAL */
    PA_ORDER_NATURAL = 1,       /* row r takes sequence r */
    PA_ORDER_LONGEST_FIRST = 2  /* row r takes the sequence with the r-th most
                                   blocks, ties by index; each work-group
                                   ranks the context lengths on the device */
};
#define PA_RANK_MAX_SEQS 256

/* How one work-group walks its blocks. */
enum pa_structure {
    PA_STRUCTURE_FUSED = 0,    /* one pass: Q.K^T, online softmax and P.V per
                                  block, with the look-ahead of whole (K, V)
                                  blocks (the default) */
    PA_STRUCTURE_TWO_LOOP = 1  /* the review's two loops (sections 3.4, 4.1):
                                  all Q.K^T with a K look-ahead, the range
                                  maximum, then all P.V with a V look-ahead.
                                  A comparison: fp16 caches only, no debug
                                  outputs, look-ahead distance 1, partitions
                                  of at most 32 blocks by default (their
                                  scores are kept in LDS) */
};

/* pa_options.even_split */
enum pa_even_split {
    PA_EVEN_SPLIT_AUTO = 0,   /* the plan's choice: the even split for 2..256
                                 sequences with at least CUs / 2 (sequence,
                                 KV head) units (E4M3 with at most 8 query
                                 heads per KV head: CUs / 4) over a table of
                                 160..1024 blocks, with waves, partitions, order and
                                 residency left to the plan, the look-ahead
                                 off or in registers, and no
                                 min_context_hint that says every context
                                 fills the table */
    PA_EVEN_SPLIT_OFF = 1,
    PA_EVEN_SPLIT_ON = 2      /* PA_ERR_UNSUPPORTED where it does not apply */
};

typedef struct pa_shape {
    int32_t num_seqs;           /* B >= 1 */
    int32_t num_q_heads;        /* Hq >= 1 */
    int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0, Hq / Hkv <= PA_G_MAX */
    int32_t head_dim;           /* must be 128 */
    int32_t block_size;         /* must be 16 */
    int32_t max_blocks_per_seq; /* row stride of block_tables, >= 1 */
    int64_t num_blocks;         /* pool size, >= 1 */
    /* Byte strides of the caches, 0 = the dense layout below.  Each (block,
       KV head) slice (4 KiB fp16, 2 KiB E4M3) must itself be laid out as
       documented; these only say where the slices are:
           K slice (p, h) at k_cache + p * k_block_stride + h * k_head_stride
           V slice (p, h) at v_cache + p * v_block_stride + h * v_head_stride
       Dense: head stride = slice bytes, block stride = num_kv_heads * that.
       Strides must be multiples of 16, head strides >= the slice bytes and
       block strides >= num_kv_heads * head stride (slices never overlap).
       One pool with K and V side by side per (block, head), for example,
       is k_head_stride = v_head_stride = 2 * slice, block strides
       num_kv_heads * 2 * slice and v_cache = k_cache + slice. */
    int64_t k_block_stride;
    int64_t k_head_stride;
    int64_t v_block_stride;
    int64_t v_head_stride;
    int32_t kv_dtype;           /* enum pa_kv_dtype; the plan (waves, LDS,
                                   default look-ahead distance) depends on it.
                                   paged_attn_decode needs PA_KV_F16 and
                                   paged_attn_decode_fp8 PA_KV_E4M3, else
                                   PA_ERR_INVALID_ARG */
} pa_shape;

typedef struct pa_options {
    int32_t prefetch;          /* enum pa_prefetch; negative = library default */
    int32_t partition_blocks;  /* blocks per split-context partition, at most
                                  1024; 0 = auto: one partition per sequence
                                  when the batch has at least as many
                                  (sequence, KV head) pairs as the device has
                                  CUs, else the balanced split (see
                                  pa_plan_info.balanced) or, when that does
                                  not apply, about CUs / pairs partitions of
                                  64..256 blocks */
    int32_t waves_per_wg;      /* w in {1, 2, 4, 8}; 0 = auto: 8 for unsplit
                                  batches of 256..767 pairs whose block table
                                  is 512..1024 blocks wide, else 4 */
    int32_t prefetch_distance; /* k, the look-ahead distance in iterations of
                                  a wave (0 = 1, or 2 for modes 2 and 4 over
                                  an E4M3 cache): mode 1 touches block j+k*w
                                  (k <= 63); mode 2 fetches block j+k*w into
                                  registers and mode 4 into LDS (k <= 2, else
                                  PA_ERR_UNSUPPORTED); mode 3 fetches j+w
                                  into registers and touches j+(1+k)*w
                                  (k <= 63).  The two-loop structure takes
                                  k = 1 only */
    int32_t seq_order;         /* enum pa_seq_order; LONGEST_FIRST needs
                                  num_seqs <= PA_RANK_MAX_SEQS */
    int32_t structure;         /* enum pa_structure */
    int32_t min_context_hint;  /* a lower bound, in tokens, on every
                                  sequence's context length, when the caller
                                  knows one (0 = none).  It only steers the
                                  plan: with a bound of at least 7/8 of the
                                  block table's width, a table of 64..1024
                                  blocks (256.. for GQA), auto waves,
                                  partitions and residency, and the
                                  look-ahead off or in registers (fp16 one
                                  block ahead, E4M3 two), the plan takes the
                                  streaming shape where it has one: for a
                                  whole number of (sequence, KV head) pairs
                                  per CU (1, 2, 3, 4 or 6 for fp16; 1 or 4
                                  for E4M3), or an fp16 balanced split with
                                  at least 256 table blocks per CU.  Its
                                  waves per
                                  work-group and residency cap keep about
                                  32 KiB of K/V loads in flight per CU from
                                  start to end.  A wrong bound changes no
                                  result, only the speed */
    int32_t max_resident_wgs;  /* at most this many decode work-groups per CU
                                  at once (0 = the plan's choice, 1..8): the
                                  launch requests the LDS that enforces it */
    int32_t even_split;        /* enum pa_even_split.  The even split gives
                                  each of S = CUs x residency work-groups an
                                  equal share of all the batch's (block, KV
                                  head) pairs, KV head 0's sequences first,
                                  then head 1's, ...; a work-group walks the
                                  pieces of the (sequence, KV head) units in
                                  its share, writes a whole unit's output
                                  directly and a piece of a unit that
                                  crosses a share boundary to the workspace,
                                  and a second kernel merges those.  The
                                  shares are found on the device from the
                                  context lengths.  It needs num_seqs <=
                                  PA_RANK_MAX_SEQS, max_blocks_per_seq <=
                                  1024, the fused structure and no explicit
                                  partition size; the sequence order does
                                  not apply */
    void *workspace;           /* device scratch for partition partials; may be
                                  NULL when the plan has one partition */
    size_t workspace_bytes;
    /* Debug outputs (all NULL in normal use; any non-NULL selects the
       checked kernel variant, which computes bitwise the same result; the
       fourth, debug_timeline, follows after them):
       debug_gather_k  fp16 [B][Hkv][max_blocks_per_seq*16][128]: the K rows
                       each wavefront actually loaded for the compute step;
       debug_trace     int32 [B][Hkv][max_blocks_per_seq][2]: per block, the
                       (wave << 16 | iteration) that computed it and the wave
                       that fetched it ahead (entries never visited keep the
                       caller's fill value);
       debug_error_word int32: bit 0 set if a block id was outside the pool,
                       bit 1 if a context length exceeded the table. */
    void *debug_gather_k;
    int32_t *debug_trace;
    int32_t *debug_error_word;
    int64_t *debug_timeline;  /* int64 [workgroups][4] (pa_plan_info.workgroups
                                 of the decode kernel): per work-group, in
                                 grid order (x fastest), its start and end on
                                 the GPU's constant 100 MHz clock
                                 (s_memrealtime) and the HW_ID and XCC_ID
                                 registers of the CU it ran on.  Work-groups
                                 with nothing to do still record both times.
                                 A debug output like the three above: the
                                 checked kernel variant runs */
} pa_options;

/* The plan a call would use, for logging and tests. */
typedef struct pa_plan_info {
    int32_t prefetch;
    int32_t waves_per_wg;
    int32_t partition_blocks;
    int32_t num_partitions;    /* partitions of the longest possible sequence */
    int64_t workgroups;        /* decode-kernel grid size */
    size_t workspace_bytes;    /* 0 when num_partitions == 1 */
    int32_t seq_order;         /* PA_ORDER_NATURAL or PA_ORDER_LONGEST_FIRST */
    int32_t structure;         /* enum pa_structure */
    int32_t prefetch_distance; /* the look-ahead distance k in effect */
    int32_t balanced;          /* 1: balanced split.  The partition size is
                                  then chosen on the device from the context
                                  lengths, per call: the smallest multiple of
                                  waves_per_wg, at least partition_blocks,
                                  with which all sequences need at most
                                  workgroups / num_kv_heads partitions (about
                                  one work-group per CU); num_partitions is
                                  the most one sequence can get.  Chosen for
                                  auto partitions when the batch has 2..256
                                  sequences and fewer (sequence, KV head)
                                  pairs than CUs, with seq_order AUTO and the
                                  fused structure */
    int32_t resident_wgs;      /* the residency cap the launch enforces
                                  (work-groups per CU), 0 = none */
    size_t lds_bytes;          /* dynamic LDS per decode work-group: what the
                                  walk needs, or more where a residency cap
                                  is enforced */
    int32_t seqs_per_wg;       /* 1, or 2: each work-group walks two
                                  sequences in turn (grid row y: ranks y and
                                  B-1-y), for 1-wave work-groups capped at 2
                                  per CU whose halved grid fills whole rounds
                                  of the cap; workgroups counts the halved
                                  grid */
    int32_t even_split;        /* 1: the even split (pa_options.even_split);
                                  workgroups = the shares; the workspace
                                  holds two partial records of Hq / Hkv rows
                                  per share and one piece record per
                                  (sequence, KV head) */
} pa_plan_info;

/* What the auto plan takes from the device.  paged_attn_plan,
   paged_attn_workspace_size and the decode calls plan for the current device,
   whose figures are queried once (hipDeviceGetAttribute: multiprocessor
   count, LDS per multiprocessor and per block) and cached per device; where
   no device can be queried the MI355X figures stand in.  A stream restricted
   to fewer CUs (a CU mask) is not seen by the query: plan such a device with
   paged_attn_plan_for_device instead of relying on the auto sizes. */
typedef struct pa_device_info {
    int32_t compute_units;           /* CUs a launch is spread over: 256 on MI355X */
    int32_t lds_bytes_per_cu;        /* LDS a CU holds: 163840 on gfx950 */
    int32_t lds_bytes_per_workgroup; /* LDS one work-group may take: 163840 on
                                        gfx950; <= lds_bytes_per_cu */
    int32_t queried;                 /* set by paged_attn_device_info: 1 if read
                                        from the device, 0 for the MI355X
                                        figures; ignored as an input */
} pa_device_info;

/* The current device's figures (or the MI355X ones, queried = 0, when there
   is none).  Host-only; never synchronises. */
int paged_attn_device_info(pa_device_info *info);

/* Fill *opts with the defaults (prefetch = library default, auto sizes). */
void paged_attn_default_options(pa_options *opts);

/* One decode step; see the conventions above.  shape must be non-NULL; opts
   may be NULL (defaults).  stream is a hipStream_t or NULL. */
int paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens,
                      float scale, void *out, const pa_shape *shape,
                      const pa_options *opts, void *stream);

/* One decode step over an FP8 KV cache (answer section 4: FP8 to shrink the
   KV footprint).  K and V hold OCP FP8 E4M3 bytes (1 sign, 4 exponent bits
   with bias 7, 3 fraction bits, no infinities, 0x7f / 0xff are NaN); a
   cached value means byte_value * k_scale (K) or * v_scale (V), both finite
   and > 0.  Layouts, one byte per value, 2 KiB per (block, KV head):
       k_cache  [num_blocks][num_kv_heads][8][16][16]
                (dim group g, token t, dim 16g+i)
       v_cache  [num_blocks][num_kv_heads][16][128]   (token, dim)
   q and out stay fp16.  The kernel widens E4M3 to fp16 exactly, applies
   k_scale to the scores and v_scale to the output, and otherwise computes
   exactly as paged_attn_decode does.  Everything else -- shape, options,
   workspace, debug outputs, status codes -- is as for paged_attn_decode;
   debug_gather_k receives the widened K bytes before k_scale. */
int paged_attn_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *block_tables, const int32_t *context_lens,
                          float scale, float k_scale, float v_scale, void *out,
                          const pa_shape *shape, const pa_options *opts, void *stream);

/* Bytes of the device scratch array that paged_attn_decode_noalloc uses in
   place of a caller's workspace (one array per GPU, held until the process
   ends). */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* paged_attn_decode for callers that cannot allocate device memory: code
   under HIP graph capture, serving loops and harnesses that forbid
   hipMalloc.  The same computation, kernels and plan as paged_attn_decode
   (bitwise the same output), except that the partition partials live in a
   library-owned device array of PA_NOALLOC_SCRATCH_BYTES on the current
   device instead of in opts->workspace, which is ignored.  The call allocates
   nothing: no hipMalloc / hipFree and no allocating library routine.
   Returns PA_ERR_WORKSPACE, before any launch, when the plan needs more
   partials than the array holds (paged_attn_workspace_size(shape, opts) >
   PA_NOALLOC_SCRATCH_BYTES), PA_ERR_HIP if the array's device address
   cannot be looked up (done once per device, on the first call there).
   Every call on one GPU shares that GPU's array, and the array keeps the
   last call's contents (nothing in it needs to start at zero: each call
   writes every partial it reads).  Calls that overlap in time on one GPU --
   on different streams, or from different host threads -- race on the array
   and give undefined results; serialise them on one stream. */
int paged_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *context_lens,
                              float scale, void *out, const pa_shape *shape,
                              const pa_options *opts, void *stream);

/* Plan for (shape, opts) on the current device without launching.
   Host-only. */
int paged_attn_plan(const pa_shape *shape, const pa_options *opts,
                    pa_plan_info *info);

/* The plan the library would make on a device with these figures
   (compute_units 1..65536, 1024 <= lds_bytes_per_workgroup <=
   lds_bytes_per_cu, else PA_ERR_INVALID_ARG).  Host-only. */
int paged_attn_plan_for_device(const pa_shape *shape, const pa_options *opts,
                               const pa_device_info *device, pa_plan_info *info);

/* Workspace bytes paged_attn_decode needs for (shape, opts); 0 if none or if
   the arguments are invalid.  Host-only. */
size_t paged_attn_workspace_size(const pa_shape *shape, const pa_options *opts);

/* K from the plain token-major layout [num_blocks][num_kv_heads][16][128]
   (token, dim; one value per element, fp16 or E4M3 bytes by kv_dtype) into
   the grouped layout paged_attn_decode / paged_attn_decode_fp8 read (see
   the layouts above): within each (block, KV head) slice, the 16-byte piece
   of token t holding dims 8g..8g+7 (fp16) or 16g..16g+15 (E4M3) moves to
   position (g, t).  A pure reindexing, bit for bit.  Both pointers are
   device pointers to dense pools, 16-byte aligned; the two ranges must not
   overlap (PA_ERR_INVALID_ARG).  Asynchronous on `stream` like the decode
   calls.  V needs no packing: its layout is the token-major one. */
int paged_attn_pack_k(const void *k_token_major, void *k_cache, int64_t num_blocks,
                      int32_t num_kv_heads, int32_t kv_dtype, void *stream);

/* Streaming-read ceiling: reads `bytes` (a multiple of 16, 16-byte aligned)
   from device buffer `buf` once, in 8 KiB chunks per wavefront of the same
   non-temporal 128-bit loads the decode kernel uses, with one 4-wave
   work-group per CU of the current device (about 32 KiB of loads in flight
   per CU, the rate-best count), and writes one 16-byte XOR per work-group
   into `sink` (device, at least paged_attn_stream_read_sink_bytes(bytes)
   bytes, 16 per CU). */
int paged_attn_stream_read(const void *buf, size_t bytes, void *sink,
                           void *stream);
size_t paged_attn_stream_read_sink_bytes(size_t bytes);

const char *paged_attn_error_string(int status);
int paged_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
