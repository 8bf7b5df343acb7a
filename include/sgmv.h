/*
 * libsgmv -- Segmented Gather Matrix-Vector multiplication (SGMV) on AMD Instinct
 * MI355X (gfx950).
 *
 * What it computes.  Punica serves many LoRA fine-tunes of one base model in one
 * batch.  The Punica project overview ("How It Works") describes a LoRA model as the
 * pretrained weight W plus two smaller matrices A and B, applied through SGMV; the
 * Punica paper summary on research.elamur.ai ("Summary", and idea I2 under
 * "Interesting ideas") says the backbone runs as one ordinary GEMM over the whole
 * batch while the per-adapter low-rank additions are computed together, with the
 * batch sorted so that requests for the same adapter are contiguous.  For every
 * token (row) t of the batch, with a = adapter_ids[t]:
 *
 *     v[t, :] = x[t, :] @ A[a]                       (shrink, h_in -> r)
 *     y[t, :] = y[t, :] + scale * v[t, :] @ B[a]     (expand, r -> h_out)
 *
 * y already holds the backbone output and is updated in place.  The backbone GEMM
 * is not part of this library.
 *
 * Conventions shared by every call:
 *   - Element type: x, y, A and B are all SGMV_F16 (IEEE binary16) or all
 *     SGMV_BF16 (bfloat16).  v and every intermediate are float32; products and
 *     sums are formed in float32 and y is rounded once, to nearest even.
 *   - x is row-major [n, h_in] with row stride ld_x elements; y is row-major
 *     [n, h_out] with row stride ld_y elements.
 *   - A[a] (h_in x r) is stored as a row-major [r, h_in] array: row j holds column
 *     j of A.  B[a] (r x h_out) is stored as a row-major [h_out, r] array: row c
 *     holds column c of B.  (This is the nn.Linear weight layout of a LoRA pair;
 *     the contracted dimension is contiguous in both.)
 *   - Segments: the batch is viewed in *sorted order*.  Sorted position i is
 *     caller row perm[i] (perm == NULL means the identity: the caller's rows are
 *     already sorted).  Segment s covers sorted positions seg_starts[s] ..
 *     seg_starts[s+1]-1 and uses adapter s of the per-segment pointer tables
 *     A_ptrs[s] / B_ptrs[s].  sgmv_build_segments / sgmv_build_ptr_table produce
 *     these tables from per-token adapter ids.
 *   - min_seg_len / max_seg_len are host-side bounds on the number of rows of any
 *     segment (sgmv_build_segments returns the exact values; 0 and n are always
 *     valid).  They only choose which kernels are launched: segments shorter than
 *     16 rows use wavefront-reduction (GEMV) kernels, longer ones MFMA tiles.
 *
 * Memory ownership: every pointer passed to a device call is device memory owned by
 * the caller, except where a comment says "host".  The library allocates no device
 * memory, keeps no per-call state and never synchronises: device calls are enqueued on
 * `stream` and return.  Calls that share a workspace must be ordered (same stream).
 * Streams (the one state the library holds): a fused call (sgmv_lora_add,
 * sgmv_lora_add_ranked, sgmv_lora_add_pool above 64 rows) whose batch has segments both
 * shorter and longer than 16 rows, or a mixed-rank call with several rank groups, made
 * while `stream` is being captured into a HIP graph, runs some of its kernel chains on
 * side streams and joins them back into `stream` before returning: the captured graph
 * orders everything after the call exactly as `stream` alone would, and its branches
 * overlap on the GPU.  Eager calls use `stream` only.  The side streams (four per device,
 * default priority, non-blocking) and their events are created by the first fused call on
 * a device that is not being captured and live until the process ends; a call captured
 * before that runs every chain on `stream`, so such a graph replays its chains one after
 * another.  A process-wide mutex keeps each fused call's fork-launch-join sequence whole
 * when host threads call concurrently.
 *
 * Errors: every argument check is done on the host before any HIP call, so a
 * rejected call has no effect.  The contents of device tables (seg_starts, perm,
 * A_ptrs, B_ptrs) are preconditions that are not checked.  n == 0 returns SGMV_OK
 * without launching anything.
 */
#ifndef SGMV_H_
#define SGMV_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGMV_ABI_VERSION 1

/* element types of x, y, A, B */
#define SGMV_F16 0
#define SGMV_BF16 1

/* status codes */
#define SGMV_OK 0
#define SGMV_ERR_NULL 1        /* a required pointer is NULL */
#define SGMV_ERR_SHAPE 2       /* a size, stride or segment bound is inconsistent */
#define SGMV_ERR_ALIGNMENT 3   /* x, y, v or an adapter base is not 16-byte aligned, or h % 8 != 0 */
#define SGMV_ERR_ADAPTER_ID 4  /* an adapter id lies outside [0, n_adapters) */
#define SGMV_ERR_UNSUPPORTED 5 /* unknown dtype, or r not in {16, 32, 64} */
#define SGMV_ERR_WORKSPACE 6   /* workspace missing, too small or not 256-byte aligned */
#define SGMV_ERR_ALIAS 7       /* an output overlaps an input */
#define SGMV_ERR_HIP 8         /* a HIP runtime call or kernel launch failed (e.g. no device) */
#define SGMV_ERR_DEVICE 9      /* sgmv_check_workspace: a device-side check set a flag bit */

/*
 * Flag bits of the workspace's first int32, set by device-side checks of calls that ran
 * on it (a set bit means some rows of some call were not computed as asked).  No kernel
 * clears them; sgmv_check_workspace reads and optionally clears them.
 */
#define SGMV_FLAG_WAIT_TIMEOUT 1 /* one-launch decode path: a bounded wait for partial sums
                                    ran out (the rows it served got wrong values) */
#define SGMV_FLAG_ADAPTER_ID 2   /* device ids: a row's id lay outside [0, n_adapters) and
                                    the row was left unchanged */
#define SGMV_FLAG_SEG_BOUNDS 4   /* host tables: a segment's length contradicted the
                                    caller's min_seg_len / max_seg_len (a long segment with
                                    max_seg_len < 16, or a short one with min_seg_len >= 16);
                                    its rows were not computed */

/* Version of this interface (SGMV_ABI_VERSION of the library that was built).  Library
 * plumbing: no passage of the pages defines it. */
int sgmv_abi_version(void);

/* Static English text for a status code; never NULL.  Library plumbing. */
const char* sgmv_status_string(int status);

/*
 * Segment metadata (host).  Stable counting sort of the caller's rows by adapter id
 * (the paper summary's idea I2: sort the batch by adapter so that each adapter's
 * requests form one dense segment).
 *   adapter_ids  host int32[n]: adapter of caller row t, in [0, n_adapters)
 *   perm         host int32[n] out: caller row at sorted position i; rows of one
 *                adapter keep their caller order
 *   seg_starts   host int32[n+1] out: first n_segments+1 entries written;
 *                seg_starts[0] = 0, seg_starts[n_segments] = n
 *   seg_adapter  host int32[n] out: adapter of segment s; segments come in
 *                ascending adapter id and adapters without rows have no segment
 *   n_segments   host out: number of distinct adapter ids present
 *   min_seg_len, max_seg_len  host out (each may be NULL): shortest and longest
 *                segment (0 when n == 0)
 * Returns SGMV_ERR_ADAPTER_ID (outputs unspecified) for an id out of range,
 * SGMV_ERR_NULL / SGMV_ERR_SHAPE for bad arguments.  n == 0 gives n_segments = 0.
 */
int sgmv_build_segments(const int32_t* adapter_ids, int32_t n, int32_t n_adapters,
                        int32_t* perm, int32_t* seg_starts, int32_t* seg_adapter,
                        int32_t* n_segments, int32_t* min_seg_len, int32_t* max_seg_len);

/*
 * One rank class of a mixed-rank batch: adapters of different ranks r in one call.  The
 * rows are grouped first by their adapter's rank, then by adapter (the paper summary's
 * idea I2, sorting the batch by adapter, with the rank as the leading key, so that each
 * rank's rows run through kernels built for that r).  The group's rows are sorted
 * positions row0 .. row0+n-1 of perm; its segments are entries seg0 .. seg0+n_segments-1
 * of seg_adapter and of the pointer tables; its segment starts, relative to row0, are
 * seg_starts[starts0 .. starts0+n_segments].
 */
typedef struct sgmv_rank_group {
  int32_t r;            /* 16, 32 or 64 */
  int32_t row0;         /* first sorted position of the group */
  int32_t n;            /* rows of the group */
  int32_t seg0;         /* first segment of the group */
  int32_t starts0;      /* index in seg_starts of the group's first start (= seg0 + the
                           group's index: each group's starts end with its own n) */
  int32_t n_segments;
  int32_t min_seg_len;  /* exact shortest / longest segment of the group */
  int32_t max_seg_len;
  float scale;          /* y += scale * ... for this group's rows; the builder writes 1 */
} sgmv_rank_group;

/*
 * Segment metadata of a mixed-rank batch (host).  Stable counting sort of the caller's
 * rows by (rank of the row's adapter, adapter id): groups in ascending r, segments in
 * ascending adapter id inside a group, rows of one adapter in caller order.
 *   adapter_ids   host int32[n]: adapter of caller row t, in [0, n_adapters)
 *   adapter_rank  host int32[n_adapters]: rank of every adapter, each in {16, 32, 64}
 *   perm          host int32[n] out: caller row at sorted position i
 *   seg_starts    host int32[n+3] out: per group, its relative starts (see
 *                 sgmv_rank_group); n_segments + n_groups entries are written
 *   seg_adapter   host int32[n] out: adapter of segment s (all groups, in order)
 *   groups        host sgmv_rank_group[3] out: the non-empty groups, ascending r
 *   n_groups      host out: number of non-empty groups (0 when n == 0)
 * Returns SGMV_ERR_ADAPTER_ID for an id out of range, SGMV_ERR_UNSUPPORTED for a rank
 * outside {16, 32, 64}, SGMV_ERR_NULL / SGMV_ERR_SHAPE for bad arguments.
 */
int sgmv_build_segments_ranked(const int32_t* adapter_ids, int32_t n, int32_t n_adapters,
                               const int32_t* adapter_rank, int32_t* perm, int32_t* seg_starts,
                               int32_t* seg_adapter, sgmv_rank_group* groups, int32_t* n_groups);

/*
 * Per-segment pointer table (host): seg_ptrs[s] = adapter_base[seg_adapter[s]].  This is
 * the "gather" of SGMV: each segment reads its own adapter's weights (paper summary,
 * "Summary": the low-rank additions of different adapters computed together in one
 * batch; project overview, "How It Works": A and B applied through SGMV).
 *   adapter_base  host uint64[n_adapters]: device address of each adapter's A (or B)
 *   seg_ptrs      host uint64[n_segments] out
 * Returns SGMV_ERR_ADAPTER_ID for an entry of seg_adapter out of range and
 * SGMV_ERR_ALIGNMENT if a referenced base is not 16-byte aligned.
 */
int sgmv_build_ptr_table(const uint64_t* adapter_base, int32_t n_adapters,
                         const int32_t* seg_adapter, int32_t n_segments, uint64_t* seg_ptrs);

/*
 * Device-side check results of the calls that ran on `workspace` (library plumbing):
 * waits for everything enqueued on `stream`, reads the workspace's flag word into *flags
 * (host; may be NULL) and, if `clear` is nonzero, resets it to zero.  Returns SGMV_OK when
 * no flag is set, SGMV_ERR_DEVICE when one is (see SGMV_FLAG_*), SGMV_ERR_HIP if the
 * stream is being captured or a copy fails.  Synchronising: not for use under capture.
 */
int sgmv_check_workspace(hipStream_t stream, void* workspace, int32_t* flags, int32_t clear);

/*
 * Bytes of device workspace that sgmv_shrink, sgmv_lora_add, sgmv_lora_add_ranked and
 * sgmv_lora_add_pool need for calls of up to n rows, h_in and rank r.  Library plumbing
 * for the shrink's split-K (v = x @ A[a] summed over K chunks, the shrink of the paper
 * summary's "Summary"): float32 split-K
 * partial sums, device-built segment tables, a few counters, and the decode path's
 * tagged partial sums, which sit at the end of the buffer.  The workspace must be 256-byte aligned and zero-filled once before its first
 * use; every call leaves it ready for the next one.  One workspace may serve any mix of
 * calls (either path, any shapes) if it is sized with the largest n, h_in and r among
 * them and the calls are stream-ordered.  Returns 0 for invalid sizes.
 */
size_t sgmv_workspace_bytes(int32_t n, int32_t h_in, int32_t r);

/*
 * Shrink only: v[i, :] = x[perm[i], :] @ A[segment of i]   (float32, sorted order): the
 * first product of the low-rank add-on x @ A @ B (project overview, "How It Works": the
 * two smaller matrices A and B; paper summary, "Summary": computed per adapter for the
 * grouped requests).
 *   v  device float32 [n, r] out, row i = sorted position i, overwritten
 * Other arguments as described above.  v must not overlap x.  A segment whose length
 * contradicts min_seg_len / max_seg_len is not computed and sets SGMV_FLAG_SEG_BOUNDS in
 * the workspace (see sgmv_check_workspace).
 */
int sgmv_shrink(hipStream_t stream, int32_t dtype, float* v,
                const void* x, int64_t ld_x, const void* const* A_ptrs,
                const int32_t* seg_starts, const int32_t* perm,
                int32_t n, int32_t n_segments, int32_t min_seg_len, int32_t max_seg_len,
                int32_t h_in, int32_t r, void* workspace, size_t workspace_bytes);

/*
 * Expand only: y[perm[i], :] += scale * v[i, :] @ B[segment of i], rounded once: the
 * second product of the low-rank add-on, added to the backbone output (project overview,
 * "How It Works"; paper summary, "Summary").
 *   v  device float32 [n, r], row i = sorted position i (as written by sgmv_shrink)
 * y must not overlap v.  This call has no workspace, so min_seg_len / max_seg_len must be
 * true bounds of the tables (sgmv_shrink on the same tables flags them if they are not).
 */
int sgmv_expand(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y, const float* v,
                const void* const* B_ptrs, const int32_t* seg_starts, const int32_t* perm,
                int32_t n, int32_t n_segments, int32_t min_seg_len, int32_t max_seg_len,
                int32_t r, int32_t h_out, float scale);

/*
 * Fused LoRA add-on: shrink then expand, y[t] += scale * (x[t] @ A[a_t]) @ B[a_t]
 * for every row, with v kept in float32 in the workspace (paper summary, "Summary": the
 * per-adapter low-rank additions of one batch computed together, same-adapter requests
 * grouped; project overview, "How It Works").  x and y must not overlap.  A segment whose
 * length contradicts min_seg_len / max_seg_len is not computed and sets
 * SGMV_FLAG_SEG_BOUNDS in the workspace (see sgmv_check_workspace).
 */
int sgmv_lora_add(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y,
                  const void* x, int64_t ld_x,
                  const void* const* A_ptrs, const void* const* B_ptrs,
                  const int32_t* seg_starts, const int32_t* perm,
                  int32_t n, int32_t n_segments, int32_t min_seg_len, int32_t max_seg_len,
                  int32_t h_in, int32_t h_out, int32_t r, float scale,
                  void* workspace, size_t workspace_bytes);

/*
 * Fused LoRA add-on for a mixed-rank batch (paper summary, "Summary": one batch mixes
 * requests of many adapters; the pages fix no common rank, so adapters of ranks 16, 32
 * and 64 may share a call): for every group g of `groups` (host array,
 * as written by sgmv_build_segments_ranked, with the scales filled in), the rows of g get
 * y[t] += g.scale * (x[t] @ A[a_t]) @ B[a_t] with A[a_t] of g.r columns.  Called eagerly,
 * the groups run one after another on `stream`, each as sgmv_lora_add on its part of the
 * tables.  Captured into a graph, with a workspace that holds every group's scratch side
 * by side (a buffer of sgmv_workspace_bytes(n, h_in, largest r) does), each
 * group's short- and long-segment kernels run on streams of their own, forked from and
 * joined back into `stream` (see "Streams" above), and overlap:
 *   A_ptrs, B_ptrs  device per-segment pointer tables over all groups' segments
 *   seg_starts      device int32: the builder's seg_starts array
 *   perm            device int32[n]: the builder's perm (required)
 *   n               rows of the batch (x and y have n rows; perm entries are < n)
 *   workspace       at least sgmv_workspace_bytes(n, h_in, largest r of the groups)
 * Every group is checked before anything is launched.  Rows that belong to no group are
 * left unchanged; x and y must not overlap.  Returns SGMV_ERR_SHAPE if a group's rows or
 * segment bounds do not fit, SGMV_ERR_UNSUPPORTED for a group rank outside {16, 32, 64}.
 */
int sgmv_lora_add_ranked(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y,
                         const void* x, int64_t ld_x, const void* const* A_ptrs,
                         const void* const* B_ptrs, const int32_t* seg_starts,
                         const int32_t* perm, int32_t n, const sgmv_rank_group* groups,
                         int32_t n_groups, int32_t h_in, int32_t h_out, void* workspace,
                         size_t workspace_bytes);

/*
 * Segment metadata on the device, for a batch of at most 4096 tokens whose adapter ids
 * are already in device memory: the same stable sort as sgmv_build_segments (paper
 * summary, idea I2), done by one wavefront for n <= 64; above, every row's sorted
 * position is its count of smaller ids plus equal ids in earlier rows (one workgroup per
 * 64 rows), then one workgroup finds and numbers the segment starts.  All pointers are
 * device memory.
 *   adapter_ids  int32[n] in; n <= 4096
 *   perm         int32[n] out (the first n_valid entries are the sorted caller rows;
 *                for n > 64 the remaining entries are set to -1)
 *   seg_starts   int32[n+1] out, seg_adapter int32[n] out
 *   n_segments   int32[1] out: S, or -1 if some id lies outside [0, n_adapters)
 *                (rows with such ids are left out of the tables)
 * Returns SGMV_ERR_SHAPE for n > 4096.  Asynchronous on `stream`.
 */
int sgmv_build_segments_device(hipStream_t stream, const int32_t* adapter_ids, int32_t n,
                               int32_t n_adapters, int32_t* perm, int32_t* seg_starts,
                               int32_t* seg_adapter, int32_t* n_segments);

/*
 * Fused LoRA add-on for adapter ids in device memory and adapters in pools,
 * y[t] += scale * (x[t] @ A[a_t]) @ B[a_t] (project overview, "How It Works"; paper
 * summary, "Summary" and idea I2: the batch grouped by adapter, each group's low-rank
 * addition computed together), with no host work that depends on the ids
 * (the call can be captured in a HIP graph and replayed with new ids):
 *   n <= 64:        one kernel launch: segment metadata, shrink and expand (decode);
 *   64 < n <= 4096: one workgroup groups the rows by adapter (a hash table in LDS; the
 *                   groups are contiguous but, unlike sgmv_build_segments_device, not in
 *                   id order) and writes the segment and pointer tables into the
 *                   workspace, then the kernels of sgmv_lora_add run on them (prefill and
 *                   mixed batches).
 *   adapter_ids  device int32[n]: adapter of caller row t (device memory, so a HIP
 *                graph can capture the call and replay it with new ids)
 *   A_pool       device: adapter a's A ([r, h_in] row-major) starts at
 *                A_pool + a * A_stride elements; A_stride >= r * h_in, multiple of 8
 *   B_pool       device: adapter a's B ([h_out, r] row-major) at B_pool + a * B_stride
 *   workspace    as for sgmv_lora_add (sgmv_workspace_bytes(n, h_in, r) bytes,
 *                zero-filled once); calls sharing a workspace must be stream-ordered
 * Rows whose id lies outside [0, n_adapters) are left unchanged and set
 * SGMV_FLAG_ADAPTER_ID in the workspace's flag word; a bounded device-side wait of the
 * one-launch kernel that ran out sets SGMV_FLAG_WAIT_TIMEOUT (the call still returns
 * SGMV_OK: it is asynchronous; sgmv_check_workspace reports both).
 * Stacked multi-layer pools: for adapters stored as [layers, P, r, h_in] (A) and
 * [layers, P, h_out, r] (B), layer l's pools are A_pool + l * P * A_stride and
 * B_pool + l * P * B_stride elements (each still 16-byte aligned); pass those with the
 * same strides, one call per layer.  Returns SGMV_ERR_SHAPE for n > 4096.
 */
int sgmv_lora_add_pool(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y,
                       const void* x, int64_t ld_x, const int32_t* adapter_ids, int32_t n,
                       const void* A_pool, int64_t A_stride, const void* B_pool,
                       int64_t B_stride, int32_t n_adapters, int32_t h_in, int32_t h_out,
                       int32_t r, float scale, void* workspace, size_t workspace_bytes);

/*
 * Fused LoRA add-on for a decode batch of at most 64 tokens whose adapter ids are in
 * HOST memory (the scheduler that forms the batch knows them), adapters in pools,
 * y[t] += scale * (x[t] @ A[a_t]) @ B[a_t] (project overview, "How It Works"; paper
 * summary, "Summary" and idea I2: the rows of one adapter are grouped inside the
 * launch, as in sgmv_lora_add_pool).  The ids are checked on the host and copied into
 * the kernel's arguments, so they reach the GPU with the launch itself: no separate
 * upload, and no load of the ids ahead of the adapter fetches.  One kernel launch.
 *   adapter_ids  HOST int32[n], each in [0, n_adapters), read before the call returns
 *   n            0 <= n <= 64
 * Every other argument, the result and the workspace are as for sgmv_lora_add_pool
 * (ids outside [0, n_adapters) are rejected on the host with SGMV_ERR_ADAPTER_ID, so no
 * row is skipped).  A graph that captures the call replays it with the ids it had when
 * captured.  Returns SGMV_ERR_SHAPE for n > 64.
 */
int sgmv_lora_add_host_ids(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y,
                           const void* x, int64_t ld_x, const int32_t* adapter_ids, int32_t n,
                           const void* A_pool, int64_t A_stride, const void* B_pool,
                           int64_t B_stride, int32_t n_adapters, int32_t h_in, int32_t h_out,
                           int32_t r, float scale, void* workspace, size_t workspace_bytes);

/*
 * On-demand adapter loading into a device adapter pool (paper summary, "Summary": the
 * runner fetches only the small LoRA matrices of an adapter when a request needs them;
 * "Key points": loading an adapter on demand takes milliseconds).
 *
 * sgmv_slot_cache (host bookkeeping, no GPU work): which adapter key occupies which slot
 * of a pool of n_slots adapters (pools laid out as for sgmv_lora_add_pool).  Not thread
 * safe: one cache per pool, used by one host thread.
 *   create   SGMV_ERR_SHAPE unless 0 < n_slots <= 2^24; *cache = NULL on failure
 *   map      keys: host int64[n] adapter keys of a batch (any values, repeats allowed);
 *            slots: host int32[n] out, the pool slot of every key.  A key that is not
 *            resident takes the lowest free slot, else the least recently used slot whose
 *            key the batch does not use (that key is evicted); each such (key, slot) is
 *            written to miss_keys / miss_slots (host, n entries) and *n_miss counts them:
 *            the caller uploads those adapters (sgmv_upload_adapter) before the SGMV call
 *            that reads them, on the same stream.  Returns SGMV_ERR_SHAPE, changing
 *            nothing, if the batch has more distinct keys than slots.
 *   lookup   *slot = the key's slot, or -1 if it is not resident
 *   evict    frees the key's slot (SGMV_ERR_ADAPTER_ID if the key is not resident)
 */
typedef struct sgmv_slot_cache sgmv_slot_cache;
int sgmv_slot_cache_create(int32_t n_slots, sgmv_slot_cache** cache);
void sgmv_slot_cache_destroy(sgmv_slot_cache* cache);
int sgmv_slot_cache_map(sgmv_slot_cache* cache, const int64_t* keys, int32_t n, int32_t* slots,
                        int64_t* miss_keys, int32_t* miss_slots, int32_t* n_miss);
int sgmv_slot_cache_lookup(const sgmv_slot_cache* cache, int64_t key, int32_t* slot);
int sgmv_slot_cache_evict(sgmv_slot_cache* cache, int64_t key);

/*
 * Upload one adapter from host memory into slot `slot` of device pools (same passages as
 * above): A_host ([r, h_in] row-major, 16-bit elements) to A_pool + slot * A_stride
 * elements and B_host ([h_out, r]) to B_pool + slot * B_stride, as two hipMemcpyAsync on
 * `stream`.  With pinned host memory (hipHostMalloc, or torch's pin_memory) the copies
 * are asynchronous; from pageable memory they return only when the data has been staged.
 * Kernels enqueued later on `stream` see the new adapter.  Host arrays must stay valid
 * until the copies complete.  Checks as for sgmv_lora_add_pool's pools, and 0 <= slot <
 * n_slots.
 */
int sgmv_upload_adapter(hipStream_t stream, void* A_pool, int64_t A_stride, void* B_pool,
                        int64_t B_stride, int32_t slot, int32_t n_slots, const void* A_host,
                        const void* B_host, int32_t r, int32_t h_in, int32_t h_out);

/*
 * Allocation-free variant of sgmv_lora_add_host_ids, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernel, arguments and result, with no workspace.  Its scratch (the
 * flag word, one counter per row and the tagged float32 partial sums) is a static device
 * array of the library, about 8.4 MB per GPU, held until the process ends; the device
 * address is looked up once per device (the current device, which `stream` must belong
 * to).  The array is zero when the library is loaded and every call that completes leaves
 * its counters and partial sums at zero again, so no clearing is needed between calls.
 * Calls on one GPU share the array: calls that overlap in time (different streams with no
 * ordering between them) race and give wrong results, so order them.  No hipMalloc,
 * hipFree or allocating library routine is called.  The flag word is not readable by the
 * caller (host ids are checked on the host; only a device-side wait that ran out, which
 * leaves wrong values, would set it).
 *   Shapes: as sgmv_lora_add_host_ids (0 <= n <= 64), and the tagged partial sums of
 *   (h_in, r), 8 * 64 * r * ceil(h_in * r / 8192) bytes, must fit 8 MiB: h_in up to
 *   524288 at r = 16, 131072 at r = 32, 32768 at r = 64.  Larger shapes return
 *   SGMV_ERR_WORKSPACE before any HIP call; other errors as sgmv_lora_add_host_ids, and
 *   SGMV_ERR_HIP if `stream` belongs to another device than the current one.
 */
int sgmv_lora_add_host_ids_noalloc(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y,
                                   const void* x, int64_t ld_x, const int32_t* adapter_ids,
                                   int32_t n, const void* A_pool, int64_t A_stride,
                                   const void* B_pool, int64_t B_stride, int32_t n_adapters,
                                   int32_t h_in, int32_t h_out, int32_t r, float scale);

#ifdef __cplusplus
}
#endif

#endif /* SGMV_H_ */
