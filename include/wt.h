/*
 * wt.h -- C ABI of the MI355X parameter-preparation library (libwt.so).
 *
 * The library implements the "parameter preparation" stage of an RL
 * weight-transfer pipeline ("Weight transfer for RL post-training in under 2
 * seconds", Perplexity, 2025; section "Task pipeline"): after a training step
 * it takes FSDP dim-0 row shards of BF16 weights, rebuilds each full tensor
 * (the full_tensor() step), fuses projections (e.g. q/k/v -> qkv,
 * gate/up -> gate_up), quantizes to FP8 and writes the bytes into a
 * registered destination region at offsets fixed ahead of time by the
 * controller's static schedule (section "Static schedule": the schedule is
 * computed once, each iteration replays it). The region stands in for the
 * remote inference GPU's memory that a one-sided RDMA WRITE would fill
 * (section "RDMA WRITE: one-sided transfers"); the destination side gets no
 * notification.
 *
 * Numerics of an FP8 output (the page lists quantization as a step but fixes
 * no format or rounding; this is the reading the library implements): OCP
 * FP8 E4M3 ("e4m3fn", max 448,
 * no infinity) with one fp32 scale per 128x128 tile of the fused tensor,
 * s = amax / 448 (s = 1 for an all-zero tile), each element
 * cast(fl32(x / s)) with IEEE-rounded fp32 division and round-to-nearest-even
 * with saturation. FP8 bytes are row-major [R x C]; scales are row-major
 * fp32 over the ceil(R/128) x ceil(C/128) tile grid. A WT_BF16_COPY output is
 * the fused BF16 bytes, unchanged.
 *
 * Conventions: every entry point returns a wt_status (no C++ exception ever
 * crosses the ABI). All pointers are plain host or device addresses; sizes
 * are in bytes unless a field says rows/cols. "stream" arguments are
 * hipStream_t values passed as void* (NULL = the null stream). Separate plans
 * are independent and may be used from different threads.
 */
#ifndef WT_H
#define WT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wt_status {
  WT_OK = 0,
  WT_E_INVAL = 1,     /* malformed task table or argument */
  WT_E_RANGE = 2,     /* a data or scale range falls outside [0, dst_bytes) */
  WT_E_OVERLAP = 3,   /* two destination ranges overlap */
  WT_E_ALIGN = 4,     /* misaligned shard pointer, BF16 dst_offset or scale_offset */
  WT_E_NOMEM = 5,     /* host or device allocation failed */
  WT_E_HIP = 6,       /* HIP runtime error; text from wt_plan_last_error() */
  WT_E_WATERMARK = 7, /* watermark below the staging need of one output */
  WT_E_STATE = 8,     /* wt_prepare already running on this plan */
  WT_E_TIMEOUT = 9    /* wt_progress_wait: the word did not reach its target in time */
} wt_status;

/* Output data type of a task (and of its fusion group). */
enum { WT_FP8_E4M3FN_B128 = 0, WT_BF16_COPY = 1 };

/* Where shards or the destination region live. */
enum { WT_MEM_DEVICE = 0, WT_MEM_PINNED_HOST = 1 };

/* How prepared bytes reach the destination region (emulated RDMA WRITE). */
enum {
  WT_DST_ZERO_COPY = 0, /* the kernels store straight into the region */
  WT_DST_STAGED = 1     /* kernels store into device staging; a copy stage moves them */
};

/* One FSDP shard: `rows` consecutive rows (row length = the task's cols,
 * BF16, row-major, rows contiguous). rows may be 0 (ptr is then ignored).
 * ptr must be 2-byte aligned. */
typedef struct wt_shard {
  const void *ptr;
  int64_t rows;
} wt_shard;

/* One task = one source parameter tensor ("Task pipeline": each parameter
 * tensor transfer is a task), given as its shards in rank order. Its full
 * tensor is the dim-0 concatenation of the shards.
 *
 * fusion_group: -1 = the task is an output of its own. Tasks that share an
 * id >= 0 form ONE output, their full tensors concatenated along dim 0 in
 * table order (projection fusion); they must share cols, dtype and
 * shard_mem, and the output's dst_offset / scale_offset are taken from the
 * group's first task (the others' offsets are ignored).
 *
 * dst_offset: byte offset of the output's data in the destination region
 * (FP8: R*C bytes; BF16 copy: 2*R*C bytes, offset must be even).
 * scale_offset: byte offset of the fp32 scale grid (FP8 only; multiple of 4).
 * A 1-D tensor of n elements is described as rows = n, cols = 1. */
typedef struct wt_task {
  const wt_shard *shards;
  int32_t n_shards;
  int32_t shard_mem; /* WT_MEM_DEVICE or WT_MEM_PINNED_HOST */
  int64_t cols;
  int32_t dtype; /* WT_FP8_E4M3FN_B128 or WT_BF16_COPY */
  int32_t fusion_group;
  uint64_t dst_offset;
  uint64_t scale_offset;
} wt_task;

/* Plan options; wt_plan_options_init() fills the defaults. */
typedef struct wt_plan_options {
  /* Upper bound on temporary device memory held by tasks in flight (the
   * watermark of the weight-transfer page's section "GPU memory usage
   * control", under which tasks are admitted). Used for staging of
   * pinned-host shards and, in WT_DST_STAGED mode, of outputs.
   * Default 512 MiB (a staged pipeline into pinned host memory with one
   * 176 MB output per layer measured 39 ms per replay under 256 MiB, 34 ms
   * under 512 MiB). */
  uint64_t watermark_bytes;
  /* Target bytes of one pipeline chunk (outputs moved through the stages
   * together, one kernel launch each). 0 (default): about 1/16 of the bytes
   * that go through the pipeline, at least 32 MiB, at most watermark / 2
   * (watermark / 3 when both shards and outputs are staged, so that each of
   * the three stages can hold a slot of the ring).
   * Smaller chunks let the first parts of the destination region complete
   * sooner (see the completion counters); many more than a few dozen chunks
   * per replay cost throughput. */
  uint64_t chunk_bytes;
  int32_t dst_write_mode; /* WT_DST_ZERO_COPY (default) or WT_DST_STAGED */
  int32_t device;         /* HIP device ordinal; -1 (default) = current device */
  /* Cache hint for reading full 128 x 128 tiles: WT_LOAD_AUTO (default; the
   * library's choice, currently non-temporal loads), WT_LOAD_PLAIN, or
   * WT_LOAD_STREAM (non-temporal loads). Affects speed only, never results;
   * values above WT_LOAD_STREAM are WT_E_INVAL. */
  uint32_t load_hint;
  /* Host-side backpressure of pipelined plans: wt_prepare first waits on the
   * host until at most max_replays_in_flight - 1 earlier replays of the plan
   * are unfinished. 0 (default): 1, i.e. a call returns once the previous
   * replay has finished and this one is enqueued. Values above 8 are
   * WT_E_INVAL. Affects speed and host blocking, never results. */
  uint32_t max_replays_in_flight;
  /* Grouping of full 128 x 128 tiles on the aligned path: WT_GROUP_AUTO
   * (default: adjacent full tiles of a row band two to a workgroup, except in
   * a launch of at most 768 full tiles, which fits in one round of
   * workgroups and is latency-bound: one tile each), WT_GROUP_SINGLE or
   * WT_GROUP_PAIR. Affects speed only, never results; values above
   * WT_GROUP_PAIR are WT_E_INVAL. */
  uint32_t tile_group;
  uint32_t reserved[3];
} wt_plan_options;

enum { WT_GROUP_AUTO = 0, WT_GROUP_SINGLE = 1, WT_GROUP_PAIR = 2 };

enum { WT_LOAD_AUTO = 0, WT_LOAD_PLAIN = 1, WT_LOAD_STREAM = 2 };

/* Shape of a plan, filled by wt_plan_check / wt_plan_get_info. */
typedef struct wt_plan_info {
  int64_t n_tasks;
  int64_t n_outputs;
  int64_t n_fp8_outputs;
  int64_t n_copy_outputs;
  int64_t n_tiles;            /* 128x128 tiles over all FP8 outputs */
  int64_t input_bytes;        /* BF16 bytes read */
  int64_t output_bytes;       /* FP8 + scale + BF16 bytes written */
  int64_t n_launches;         /* kernel launches per wt_prepare */
  int64_t n_chunks;           /* pipeline chunks (0 when no stage needs staging) */
  int64_t n_h2d_copies;       /* host-to-device copies per wt_prepare */
  int64_t n_dst_copies;       /* staging-to-destination copies per wt_prepare */
  int64_t staging_bytes;      /* device staging allocated (<= watermark) */
  int64_t n_units;            /* completion units: the device-resident launch (if any), then each chunk */
  int64_t n_regular_items;    /* work items of full tiles on the aligned path (a pair of tiles is one item) */
  int64_t n_edge_tiles;       /* aligned-path tiles that are partial or draw rows from several shards */
  int64_t n_general_tiles;    /* tiles of outputs with ragged columns or unaligned addresses */
} wt_plan_info;

/* One operation of the replayed schedule, as listed by wt_plan_schedule. */
typedef struct wt_sched_op {
  int32_t stage;        /* 0 = host-to-device copy, 1 = prepare launch, 2 = destination copy */
  int32_t chunk;        /* chunk index (-1: the launch over device-resident outputs) */
  int32_t wait_chunk;   /* stage 0: chunk whose release this op waits for (-1: none) */
  int32_t reserved;
  int64_t bytes;        /* bytes moved (stages 0, 2) or prepared input bytes (stage 1) */
  int64_t staging_offset; /* start of the chunk's staging slot in the ring */
  int64_t staging_bytes;  /* size of the chunk's staging slot */
} wt_sched_op;

typedef struct wt_plan wt_plan;

/* Fills `opts` with the defaults. */
void wt_plan_options_init(wt_plan_options *opts);

/* Validates a task table exactly as wt_plan_create does and describes the
 * plan it would build, without touching any GPU (host only). opts may be
 * NULL (defaults). info may be NULL. */
wt_status wt_plan_check(const wt_task *tasks, size_t n_tasks, size_t dst_bytes, int32_t dst_kind,
                        const wt_plan_options *opts, wt_plan_info *info);

/* Lists the operations one wt_prepare would enqueue, in enqueue order, for
 * the plan wt_plan_check would build (host only). Writes at most max_ops
 * records to ops (may be NULL) and the total count to *n_ops. */
wt_status wt_plan_schedule(const wt_task *tasks, size_t n_tasks, size_t dst_bytes, int32_t dst_kind,
                           const wt_plan_options *opts, wt_sched_op *ops, size_t max_ops, size_t *n_ops);

/* Builds a plan: the static schedule of "Weight transfer for RL post-training
 * in under 2 seconds", section "Static schedule" (the transfer schedule is
 * computed once at initialisation and every training step replays it). It
 * validates the table,
 * builds the device descriptor tables (outputs, row segments, tile and copy
 * work lists), allocates staging within the watermark and creates the
 * plan's streams and events. The table is copied; the caller may free it on
 * return. Shard memory and the destination region stay owned by the caller
 * and must outlive the plan; their ADDRESSES are fixed in the plan, their
 * CONTENTS may change between wt_prepare calls.
 * dst: destination region base (device pointer, or pinned host pointer when
 * dst_kind is WT_MEM_PINNED_HOST), dst_bytes long. On failure *out is NULL. */
wt_status wt_plan_create(const wt_task *tasks, size_t n_tasks, void *dst, size_t dst_bytes, int32_t dst_kind,
                         const wt_plan_options *opts, wt_plan **out);

/* For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): builds the same plan
 * as wt_plan_create, with the same arguments, validation and results, but
 * calls no hipMalloc, hipHostMalloc or hipFree (host-side bookkeeping uses
 * the C++ heap). Its device descriptor tables go into a static array of
 * WT_NOALLOC_TABLE_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends; they are copied there synchronously before
 * the call returns. Limits:
 *  - one such plan per device at a time: while one is live on the device,
 *    another call returns WT_E_STATE (destroy the first with
 *    wt_plan_destroy, which waits for its latest wt_prepare launch);
 *  - tables larger than WT_NOALLOC_TABLE_BYTES (16 MiB): WT_E_NOMEM. A pair
 *    of full 128 x 128 tiles takes 32 bytes of tables, so 16 MiB holds, for
 *    example, a dense 7B-shaped model (about 6.5 MB of tables);
 *  - pinned-host shards or WT_DST_STAGED (they need staging memory):
 *    WT_E_INVAL.
 * Replays, progress words and destruction work as for any plan. A plan
 * created here shares the device's array with every later one: a graph that
 * captured its replays must not be launched after it is destroyed, and work
 * of an earlier plan that still reads the array when a new plan is created
 * (graph launches are not tracked) races with it. */
#define WT_NOALLOC_TABLE_BYTES 16777216u
wt_status wt_plan_create_noalloc(const wt_task *tasks, size_t n_tasks, void *dst, size_t dst_bytes,
                                 int32_t dst_kind, const wt_plan_options *opts, wt_plan **out);

/* Replays the plan (same page, section "Static schedule": each iteration
 * replays the schedule; section "Task pipeline": per task, the stages
 * parameter preparation -> RDMA transfer, each with its own FIFO queue, a
 * task moving to the next queue once its stage is done). Enqueues the whole
 * preparation so that it is ordered
 * after prior work on `stream` and completes before later work on `stream`.
 * With device-resident shards and WT_DST_ZERO_COPY this is one kernel launch
 * on `stream`. Pinned-host shards or WT_DST_STAGED run the three-stage
 * pipeline (host-to-device copy, prepare, destination copy) on the plan's own
 * streams, one in-order queue per stage, and join `stream` at the end.
 * Returns without waiting for the GPU, except that a pipelined plan keeps at
 * most max_replays_in_flight replays enqueued and unfinished: by default a
 * call first waits on the host for the plan's previous replay (deeper queues
 * of copies make the runtime block single copy submissions in lockstep with
 * the GPU and starve the copy engine). No validation or allocation
 * happens here. A plan without a pipeline may be replayed inside stream
 * capture (its launches, completion-word kernels and event record become
 * graph nodes; each graph replay is a replay of the plan); a pipelined plan
 * may not, since its backpressure waits on the host (WT_E_STATE, nothing
 * enqueued). A graph holding captured replays reads the plan's device
 * tables every time it is launched: it must not be launched after
 * wt_plan_destroy, and its launches must have finished before that call.
 * Returns WT_E_STATE if another wt_prepare on the same plan is
 * running in another thread, WT_E_HIP on a runtime error. */
wt_status wt_prepare(wt_plan *plan, void *stream);

/* Copies the plan's shape into *info. */
wt_status wt_plan_get_info(const wt_plan *plan, wt_plan_info *info);

/* Ends a plan. The staging it frees is the temporary memory that the
 * watermark bounds ("Weight transfer for RL post-training in under 2
 * seconds", section "GPU memory usage control"). Waits for the plan's work
 * already enqueued (its own streams, and for a plan without a pipeline the
 * latest wt_prepare launch on the caller's stream), then frees everything
 * the plan owns (device tables, staging, streams, events). Launches of a
 * captured graph are not waited for: every graph holding replays of this
 * plan must have finished, and must not be launched again, before this
 * call. Never frees shards or the destination region. NULL is ignored. */
void wt_plan_destroy(wt_plan *plan);

/* Static text for a status code. */
const char *wt_status_str(int status);

/* Text of the last error recorded on `plan`, or, for plan == NULL, of the
 * last failed wt_plan_create / wt_plan_check on the calling thread. */
const char *wt_plan_last_error(const wt_plan *plan);

/* ---- Element-function checks (exhaustive verification of the kernels' arithmetic) ----
 * These run the same device code the prepare kernel runs per tile and per
 * element, over complete input domains, so that the result can be compared
 * with an independent implementation. */

/* out[i * 65536 + x] = E4M3 byte that the prepare kernel writes for the BF16
 * pattern x in a tile whose amax is the BF16 pattern amax_bits[i] (the sign
 * bit of amax_bits is ignored; scale and division chosen exactly as in the
 * prepare kernel). path = 0: the element function of the aligned (fast) tile
 * path; path = 1: that of the general (any shape, any alignment) tile path.
 * amax_bits and out are device pointers; out holds n_amax * 65536 bytes;
 * 0 <= n_amax <= 2^20 (WT_E_INVAL otherwise). */
wt_status wt_quantize_domain(const uint16_t *amax_bits, int64_t n_amax, int32_t path, uint8_t *out, void *stream);

/* out[i] = the kernel's fp32 -> E4M3 cast of the fp32 bit pattern first + i
 * (wrapping modulo 2^32), for i < count. out is a device pointer. */
wt_status wt_cast_f32_range(uint32_t first, uint64_t count, uint8_t *out, void *stream);

/* ---- Static schedule builder (host only) ----
 * The controller's computation ("Weight transfer for RL post-training in
 * under 2 seconds", section "High-level workflow": collect parameter
 * metadata from training and inference, compute a static transfer schedule
 * that says which training GPU sends which parameter where and in what
 * order; section "Static schedule": computed once, replayed every step).
 * Input: the training side's parameters (unique names, full shapes, FSDP
 * dim-0 shard count and, optionally, shard addresses) and the inference
 * side's tensors (names, the training parameters fused into each, in fusion
 * order, and the output dtype). Output: destination offsets packed in the
 * order of the inference tensors (data, then the FP8 scale grid, each
 * aligned), the source GPU of every output (longest-processing-time-first
 * over BF16 input bytes; ties to the lower index), and the task table that
 * wt_plan_create takes, for all sources or one. Shards are the torch.chunk
 * split of the rows: ceil(rows / n) rows each, trailing shards smaller or
 * empty. */

typedef struct wt_param_meta {
  const char *name;              /* unique, NUL-terminated */
  int64_t rows, cols;            /* full shape; a 1-D tensor of n elements is rows = n, cols = 1 */
  int32_t n_shards;              /* FSDP dim-0 shards, >= 1 */
  int32_t shard_mem;             /* WT_MEM_DEVICE or WT_MEM_PINNED_HOST */
  const void *const *shard_ptrs; /* n_shards addresses, or NULL (tasks then carry NULL shard pointers) */
} wt_param_meta;

typedef struct wt_dst_meta {
  const char *name;              /* inference-side tensor name */
  const char *const *components; /* training parameter names, in fusion (dim-0 concatenation) order */
  int32_t n_components;          /* >= 1; all components must have the same cols */
  int32_t dtype;                 /* WT_FP8_E4M3FN_B128 or WT_BF16_COPY */
} wt_dst_meta;

typedef struct wt_schedule_options {
  uint64_t align;    /* destination offset alignment, a power of two >= 16; 0 = 256 */
  int32_t n_sources; /* source GPUs to balance outputs over; 0 = 1 */
  int32_t reserved[5];
} wt_schedule_options;

typedef struct wt_schedule wt_schedule;

/* Matches names, validates (unknown or duplicate names, cols that differ
 * inside a fusion group, rows < 1: WT_E_INVAL), packs offsets and assigns
 * sources. The inputs are copied. On failure *out is NULL and
 * wt_plan_last_error(NULL) says why. */
wt_status wt_schedule_build(const wt_param_meta *params, size_t n_params, const wt_dst_meta *dsts, size_t n_dsts,
                            const wt_schedule_options *opts, wt_schedule **out);

/* Totals: tasks (one per fusion component) and shard records over all
 * sources, the destination region size, and how many training parameters no
 * inference tensor uses. Any pointer may be NULL. */
wt_status wt_schedule_info(const wt_schedule *sch, size_t *n_tasks, size_t *n_shards, uint64_t *dst_bytes,
                           size_t *n_unused_params);

/* Placement of inference tensor i: data and scale offsets (scale_offset is
 * 0 for BF16 copies), its source GPU and its BF16 input bytes. */
wt_status wt_schedule_output(const wt_schedule *sch, size_t i, uint64_t *dst_offset, uint64_t *scale_offset,
                             int32_t *source, uint64_t *input_bytes);

/* Writes the task table of one source (source = -1: every source) in
 * inference-tensor order: tasks[0 .. *n_tasks) with their shard records in
 * shards[]; task.shards points into the caller's shards array. Fusion
 * groups are numbered by inference-tensor index. WT_E_RANGE if max_tasks or
 * max_shards is too small (*n_tasks and *n_shards_out then give the sizes
 * needed). */
wt_status wt_schedule_tasks(const wt_schedule *sch, int32_t source, wt_task *tasks, size_t max_tasks,
                            wt_shard *shards, size_t max_shards, size_t *n_tasks, size_t *n_shards_out);

/* Frees the schedule. NULL is ignored. */
void wt_schedule_destroy(wt_schedule *sch);

/* ---- Block-scaled FP8 quantization of token activations ----
 * The sender half of MoE dispatch quantizes token activations to FP8 with
 * block scales before writing them to peers ("Enabling trillion-parameter
 * models on AWS EFA", dispatch/combine evaluation: hidden size 7168, FP8
 * dispatch with block scales; the sender shuffles tokens into send buffers
 * so each peer receives one write). Blocks are 1 x 128: one token's 128
 * consecutive channels, the last block of a row holding cols % 128 channels
 * when cols is not a multiple of 128. Per block s = amax / 448 in IEEE fp32
 * (1 for an all-zero block) and q = E4M3(fl32(x / s)), round to nearest even,
 * saturating: the same arithmetic as the weight tiles.
 *
 * x: n_rows rows of BF16 on the device, x_row_stride elements apart (>= cols),
 *    2-byte aligned.
 * row_index: NULL, or n_out int32 input-row indices on the device: output
 *    row i quantizes input row row_index[i] (row i when NULL). Output rows
 *    whose index is outside [0, n_rows) are not written. Indices may repeat.
 * q: n_out rows of q_row_stride bytes (>= cols), device or pinned host; the
 *    first cols bytes of a row receive the FP8 codes, the rest is untouched.
 * scales: n_out rows of scale_row_stride bytes (>= 4 ceil(cols / 128)),
 *    4-byte aligned, device or pinned host; the row's block scales as fp32.
 *    q and scales may interleave (e.g. one send-buffer slot per token holding
 *    its codes, then its scales) as long as no two written ranges overlap.
 * Shapes with cols, x_row_stride and q_row_stride multiples of 8, x 16-byte
 * and q 8-byte aligned take the vector path; any other shape takes a general
 * path with the same results.
 * Enqueued on `stream` (a hipStream_t; NULL = the default stream); returns
 * without waiting. Errors: WT_E_INVAL for negative or inconsistent sizes,
 * NULL pointers with n_out > 0, n_out * ceil(cols / 128) >= 2^31 or
 * cols >= 2^31; WT_E_ALIGN for a misaligned x or scales; WT_E_HIP if the
 * launch fails. Pointer kinds and extents are not queried (that would cost a
 * runtime call per pointer per call on the dispatch path): the caller
 * guarantees that every range above lies in its allocation. n_out == 0 is a
 * no-op. */
wt_status wt_quantize_act_b128(const void *x, int64_t n_rows, int64_t cols, int64_t x_row_stride,
                               const int32_t *row_index, int64_t n_out, void *q, int64_t q_row_stride,
                               void *scales, int64_t scale_row_stride, void *stream);

/* ---- Completion counters ----
 * Host-visible words that the GPU writes as parts of a replay finish, so a
 * host thread can start moving a part of the destination region (the one-sided
 * write to the inference side) as soon as it is final instead of waiting for
 * the whole replay ("RDMA point-to-point communication for LLM systems",
 * GPU-progress notification through memory words that kernels update and the
 * CPU polls; receiver-side counters per index). A replay finishes in units: the
 * launch over device-resident outputs (unit 0 when the plan has one), then
 * each pipeline chunk in order; wt_plan_info.n_units counts them and
 * wt_plan_task_unit maps a task to its unit. */

/* Attaches `words` (n_words >= n_units 8-byte words in pinned host memory,
 * 8-byte aligned; owned by the caller, who must keep it alive while the plan
 * replays) to the plan and resets the plan's replay counter. From then on the
 * r-th wt_prepare (r = 1, 2, ...) stores r into words[u] once every byte of
 * unit u is in the destination region: after the unit's prepare launch
 * (zero-copy) or after its destination copies (WT_DST_STAGED). The stores are
 * made by a one-thread kernel on the stream that ran the unit, with release
 * ordering at system scope, behind the unit's work. Passing words == NULL
 * detaches. Call only while no replay of this plan is in flight. The words are
 * never cleared by the library. WT_E_INVAL for a short, misaligned or
 * non-pinned array. */
wt_status wt_plan_set_progress(wt_plan *plan, uint64_t *words, size_t n_words);

/* *unit = the completion unit that covers task `task` (index into the table
 * given to wt_plan_create). WT_E_INVAL if task is out of range. */
wt_status wt_plan_task_unit(const wt_plan *plan, size_t task, int32_t *unit);

/* Host-side wait: polls *word (acquire loads) until it is >= target or
 * timeout_ns elapses. WT_OK when reached (the unit's bytes are then visible to
 * the host), WT_E_TIMEOUT otherwise, WT_E_INVAL for a NULL word. Makes no HIP
 * call. */
wt_status wt_progress_wait(const uint64_t *word, uint64_t target, uint64_t timeout_ns);

#ifdef __cplusplus
}
#endif

#endif /* WT_H */
