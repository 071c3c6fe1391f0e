/*
 * mbk.h -- C ABI of libmbk: one batch-1 decode step of a pre-norm Llama-style
 * decoder, run on an AMD MI355X (gfx950) as ONE persistent kernel launch.
 *
 * What a step computes (MegaBake article, "What a megakernel is, and why
 * small models want one": per layer RMSNorm, Q/K/V projections, RoPE,
 * attention, output projection, residual add, RMSNorm, gate and up
 * projections, SiLU, down projection, residual add; MegaBake README mirror,
 * "Current status": the kernel also covers the embedding, the final norm, the
 * vocabulary projection and the KV-cache update), followed by a greedy
 * argmax of the logits.
 *
 * Conventions shared by every entry point
 *  - All functions return an int status: MBK_OK (0) or one of MBK_ERR_*.
 *    mbk_last_error() returns a thread-local message for the last failure.
 *  - Device buffers (source weights, packed weights, KV cache, workspace,
 *    logits, argmax) are owned by the caller and passed as raw device
 *    pointers; the library never frees them and allocates no device memory
 *    on the decode path.  Streams are hipStream_t passed as void*.
 *  - Validation happens on the host before any HIP call: a call that returns
 *    MBK_ERR_ARG / RANGE / SIZE / UNSUPPORTED / STATE has launched nothing.
 *  - One handle per stream; calls on one handle are not reentrant.
 *  - Like the README's strict default (section "The compilation path":
 *    compilation errors rather than falling back), an unsupported shape is an
 *    error, never a slower path.
 */
#ifndef MBK_H
#define MBK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MBK_OK = 0,
    MBK_ERR_ARG = 1,         /* NULL pointer, token outside [0, vocab), bad enum */
    MBK_ERR_RANGE = 2,       /* position outside [0, kv_capacity) */
    MBK_ERR_SIZE = 3,        /* caller buffer smaller than required */
    MBK_ERR_UNSUPPORTED = 4, /* dimensions the kernels do not handle */
    MBK_ERR_HIP = 5,         /* a HIP runtime call failed (message has the HIP error) */
    MBK_ERR_TIMEOUT = 6,     /* a bounded wait (input poll or grid barrier) expired on the device */
    MBK_ERR_STATE = 7        /* call made before mbk_pack_weights / mbk_alloc_kv */
};

/* Pass as `token` to reuse the previous step's device-side argmax, so a greedy
 * loop needs no host round trip (the README's "pipelined calls"). */
#define MBK_TOKEN_PREV (-1)

/* How the intervals of the persistent kernel are ordered (mbk_set_sync_mode).
 * DATAFLOW (default): every activation handed between intervals is written as
 *   8-byte {value, tag} entries and each workgroup polls exactly the entries
 *   it reads, without grid barriers (the MegaBake article's roadmap, section
 *   "Checking the 5.5x": per-phase event counters instead of grid barriers).
 * BARRIER: a counting grid barrier closes every interval (the article's
 *   "How a model gets in" executor).  Both give bitwise identical results. */
enum { MBK_SYNC_DATAFLOW = 0, MBK_SYNC_BARRIER = 1 };

/* Decoder shape. Supported: head_dim in {16, 32, 64, 128}; n_heads a multiple
 * of n_kv_heads with n_heads / n_kv_heads <= 8; hidden, n_heads*head_dim and
 * intermediate multiples of 8 and <= 8192; kv_capacity <= 8192 (the README's
 * bound on decode KV state, "Current status"). */
typedef struct {
    int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab, kv_capacity;
    int32_t qkv_bias; /* 0 or 1: bias added to the Q/K/V projections */
    float rms_eps, rope_theta;
} mbk_config;

/* Source weights: bf16 device pointers in Hugging Face layout (row-major
 * [out][in]).  Per-layer fields are HOST arrays of n_layers device pointers.
 * The LM head is the tied embedding.  bq/bk/bv are read only if qkv_bias. */
typedef struct {
    const void *embed;      /* [vocab][hidden] */
    const void *final_norm; /* [hidden] */
    const void *const *attn_norm, *const *wq, *const *wk, *const *wv;
    const void *const *bq, *const *bk, *const *bv;
    const void *const *wo, *const *mlp_norm, *const *wgate, *const *wup, *const *wdown;
} mbk_weights;

typedef struct mbk_model mbk_model; /* opaque host handle */

/* Validates the shape and creates a handle. No device work.
 * Passage: the MegaBake README mirror, "The compilation path" (strict
 * compilation: a shape outside what the bodies handle is an error,
 * MBK_ERR_UNSUPPORTED, not a fallback) and "Current status" (the limits it
 * lists: bf16, static shapes, decode KV capacity <= 8,192).
 * Errors: MBK_ERR_ARG (null pointer, a non-positive dimension, eps or theta,
 * qkv_bias not 0/1), MBK_ERR_UNSUPPORTED (a shape outside the list above).
 * *out receives a handle the caller releases with mbk_destroy. */
int mbk_create(const mbk_config *cfg, mbk_model **out);

/* Frees the handle only (never caller memory). NULL is a no-op.  Makes a HIP
 * call only when the ablation's hipGraph was instantiated (it is destroyed
 * here), so release handles before the process tears the HIP runtime down.
 * Passage: none on the pages; this repository's host-side design. */
void mbk_destroy(mbk_model *m);

/* Packs the weights into the streaming layout the kernels read.
 * Passage: none on the pages defines a packed layout (the article, "How a
 * model gets in", step 3, has the GEMM body read weight tiles directly; the
 * article's "What a megakernel is" fixes what is read: every weight once per
 * token, ~269 MB for SmolLM-135M).  The layout is this repository's design.
 * dst == NULL: writes the required size to *dst_bytes and returns.
 * Otherwise packs device-to-device on `stream` into dst (>= *dst_bytes bytes,
 * 256-byte aligned); the handle keeps dst, which the caller keeps alive.
 * src: bf16 device pointers, each 16-byte aligned, read only; the call
 * synchronises `stream` before it returns, so src may be freed afterwards.
 * Every matrix is stored as tiles of RT rows in which each wave-wide 16-byte
 * load reads 1 KiB of contiguous memory.  The payload is 2 bytes per
 * parameter plus the zero rows padding the last tile of a matrix and, where
 * the planner widens a matrix with few tiles to one row per tile, zero
 * input groups up to a multiple of 512 inputs (at most 15 % of that matrix:
 * the Qwen2-0.5B-shaped output projection gains 14 %).  Also builds the fp32
 * RoPE table and the schedule (interval table, task lists) inside dst.
 * Errors: MBK_ERR_ARG (null or misaligned pointer), MBK_ERR_SIZE (dst too
 * small), MBK_ERR_UNSUPPORTED (no schedule fits the device), MBK_ERR_HIP. */
int mbk_pack_weights(mbk_model *m, const mbk_weights *src, void *dst, size_t *dst_bytes, void *stream);

/* Where one packed matrix sits in the blob of mbk_pack_weights, so callers
 * (and tests) can read the packed layout.  Passage: none on the pages; this
 * repository's layout.  A matrix of `rows` rows (in packed order) and `cols`
 * inputs is stored as `tiles` tiles of rows_per_tile rows; each row's inputs
 * are cut in 8-element groups spread over lanes_per_row = 64 / rows_per_tile
 * lanes, and the 16-byte group of packed row t * rows_per_tile + l /
 * lanes_per_row, group (l % lanes_per_row) + s * lanes_per_row sits at byte
 * offset + ((t * steps + s) * 64 + l) * 16 for bf16 (s < steps; groups from
 * cols / 8 on, and rows from `rows` on, are zero).  kind 0: packed row r is source row
 * r; kind 1 (Q/K/V): rows [0, n_heads * head_dim) are queries, then keys, then
 * values, and inside each query or key head packed rows 2m, 2m + 1 are head
 * dims m, m + head_dim / 2; kind 2 (gate/up): packed row 2i is gate row i and
 * 2i + 1 up row i.  which: 0 Q/K/V, 1 output projection, 2 gate/up, 3 down
 * projection of `layer`; layer = -1, which = 0: the embedding table the row
 * gather reads (always bf16), which = 1: the vocabulary projection (that same
 * table, or its fp8 copy).  format 0: bf16 groups of values_per_group = 8;
 * format 1 (mbk_set_weight_format): groups of 16 E4M3 codes, and each tile
 * of tile_bytes bytes ends with the fp32 scales of its rows_per_tile rows at
 * byte scale_offset of the tile (16-byte padded, padding zero; a padding
 * row's scale is 0).  In general the group above sits at byte offset +
 * t * tile_bytes + (s * 64 + l) * 16, and groups from cols / values_per_group
 * on are zero.
 * Errors: MBK_ERR_ARG (null pointer), MBK_ERR_RANGE (layer or which out of
 * range), MBK_ERR_UNSUPPORTED / MBK_ERR_HIP as when planning. */
typedef struct {
    uint64_t offset;
    int32_t rows, cols, lanes_per_row, rows_per_tile, steps, tiles, kind;
    int32_t format, values_per_group, tile_bytes, scale_offset;
} mbk_matrix_layout;
int mbk_get_matrix_layout(mbk_model *m, int32_t layer, int32_t which, mbk_matrix_layout *out);

/* Binds the KV cache and the workspace.
 * Passage: the project site, "Integration & evaluation" (bounded contiguous
 * decode KV state), and the README mirror, "Current status" (the kernel
 * performs the KV-cache updates; decode KV capacity <= 8,192).  The
 * workspace (tagged activations, barrier and merge counters) is this
 * repository's design.
 * kv == NULL or ws == NULL: writes the required sizes and returns.
 * Otherwise zero-fills both on `stream` and keeps them.
 * KV layout: bf16 [n_layers][2 (K, V)][n_kv_heads][kv_capacity][head_dim],
 * keys stored after rotation; callers may pre-fill slots through this layout.
 * Both buffers must be 256-byte aligned. */
int mbk_alloc_kv(mbk_model *m, void *kv, size_t *kv_bytes, void *ws, size_t *ws_bytes, void *stream);

/* One decode step at position `pos` (0-based) for `token`, asynchronous on
 * `stream`.  Passage: the MegaBake article, "What a megakernel is, and why
 * small models want one" (the per-layer operations, in order) and "How a
 * model gets in" (one persistent launch walking a table of phases); the
 * README mirror, "Current status" (embedding, final norm, vocabulary
 * projection and KV update inside the kernel; flash-decoding attention); the
 * project site, "Decode leaderboard" (batch 1, one token per call).
 * Writes KV slot `pos` of every layer, attends positions 0..pos,
 * writes fp32 logits[vocab] (if logits != NULL) and the greedy argmax
 * (lowest index among equal maxima) to argmax[0] (device int32).  Re-running
 * a step at the same pos overwrites slot pos before reading it.
 * One launch of one workgroup per CU (plain by default; see
 * mbk_set_launch_mode). */
int mbk_decode_step(mbk_model *m, int32_t token, int32_t pos, float *logits, int32_t *argmax, void *stream);

/* Multi-token prefill: runs the decoder over the n_tokens prompt tokens at
 * positions pos0 .. pos0 + n_tokens - 1 at once, writing their KV-cache slots
 * (every layer), and the fp32 logits[vocab] (if logits != NULL) and greedy
 * argmax (argmax[0], device int32) of the last position; a following
 * mbk_decode_step with MBK_TOKEN_PREV continues from that argmax.  Equal, to
 * rounding, to n_tokens decode steps at those positions.  The projections
 * run as matrix-core GEMMs over the packed weights, bf16 or fp8 (activations
 * as hi/lo bf16 pairs, ~16 significant bits, fp32 accumulation); attention is causal over
 * cache slots 0 .. pos0 + i for prompt position i, in fp32.  Passage: the
 * MegaBake third-party article, "Where it breaks today" (prefill through the
 * decode-shaped bodies is slow above ~64 tokens) and the project site, "Next"
 * (fast long-prompt prefill).
 * tokens: HOST array of n_tokens ids in [0, vocab) (copied before the call
 * returns).  scratch: caller device buffer, 256-byte aligned, of at least
 * mbk_prefill_scratch_bytes(n_tokens) bytes.  Needs packed weights and a
 * bound KV cache (MBK_ERR_STATE).  Asynchronous on `stream`.
 * Errors: MBK_ERR_ARG (null pointer, n_tokens < 1, a token out of range),
 * MBK_ERR_RANGE (positions outside the cache), MBK_ERR_SIZE (scratch too
 * small), MBK_ERR_HIP. */
int mbk_prefill(mbk_model *m, const int32_t *tokens, int32_t n_tokens, int32_t pos0, void *scratch,
                size_t scratch_bytes, float *logits, int32_t *argmax, void *stream);

/* Scratch bytes mbk_prefill needs for n_tokens tokens (no device work).
 * Passage: none on the pages; this repository's buffer contract.
 * MBK_ERR_RANGE when n_tokens exceeds the cache. */
int mbk_prefill_scratch_bytes(mbk_model *m, int32_t n_tokens, size_t *bytes);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the step of
 * mbk_decode_step with the library's static scratch as its workspace, so no
 * workspace is bound and nothing is allocated.  Same kernels and bitwise the
 * same logits, argmax and cache contents as mbk_decode_step.
 * kv: the caller's cache in the layout of mbk_alloc_kv (bf16
 * [n_layers][2][n_kv_heads][kv_capacity][head_dim], 256-byte aligned),
 * read and written at slot pos; mbk_alloc_kv is not needed.  Needs packed
 * weights (MBK_ERR_STATE).  The scratch is a file-scope device array of
 * 512 KiB; each GPU the library runs on holds its own copy until the process
 * ends.  A shape whose workspace exceeds it is rejected with MBK_ERR_SIZE
 * before anything runs (every shape up to the SmolLM-1.7B one fits: 296 KB).
 * Every handle on a GPU shares that GPU's scratch: calls that overlap on one
 * GPU (two streams, two threads) race, and MBK_TOKEN_PREV reads the argmax of
 * the last static step on the GPU, whichever handle ran it.  The scratch is
 * cleared (by a kernel, not a memset) on first use and after mbk_check has
 * reported MBK_ERR_TIMEOUT for it; its activation tags never repeat between
 * clears.  Errors otherwise as mbk_decode_step. */
int mbk_decode_step_static(mbk_model *m, void *kv, int32_t token, int32_t pos, float *logits, int32_t *argmax,
                           void *stream);

/* Same bodies and results (bitwise), one kernel launch per interval
 * (the per-operator ablation).  use_graph = 1 replays the launches as a
 * hipGraph instantiated once per handle (re-instantiated when logits or
 * argmax change).  Passage: the MegaBake article, "What a megakernel is, and
 * why small models want one" (separate launches, and CUDA graphs that replay
 * them with a small gap between kernels, as the alternative to one launch).
 * Errors as mbk_decode_step. */
int mbk_decode_step_ablation(mbk_model *m, int32_t token, int32_t pos, float *logits, int32_t *argmax,
                             int32_t use_graph, void *stream);

/* Synchronises `stream` and reports device-side errors (MBK_ERR_TIMEOUT
 * when a bounded wait expired; the KV/workspace must then be re-bound with
 * mbk_alloc_kv).  Passage: none on the pages (their barrier waits are
 * unbounded); the bounded waits and this report are this repository's
 * failure detection. */
int mbk_check(mbk_model *m, void *stream);

/* Grid-barrier microbenchmark: one cooperative launch running n barriers with
 * empty bodies; *us_per_barrier = (t(n) - t(0)) / n from HIP events.
 * Passage: the MegaBake article, "How a model gets in" (the counting grid
 * barrier: one release-add per block, acquire loads until the count reaches
 * (ordinal + 1) * workers) and the README mirror, "Current status" (its cost
 * at 60 blocks).  Needs packed weights and a bound workspace (MBK_ERR_STATE);
 * n > 0 (MBK_ERR_ARG). */
int mbk_barrier_bench(mbk_model *m, int32_t n, void *stream, float *us_per_barrier);

/* Grid-barrier validation: one cooperative launch running n rounds; in round
 * i every workgroup writes i into its own epoch slot, passes the counting
 * grid barrier, then reads every workgroup's slot, which must hold at least
 * i.  first_bad (4 host int32): {round, reader workgroup, writer workgroup,
 * value read} of the first failed check, round = 0 when every check of every
 * round passed.  Passage: the MegaBake article, "How a model gets in" (the
 * counting grid barrier whose correctness every interval relies on).  Needs
 * packed weights and a bound workspace (MBK_ERR_STATE); n > 0
 * (MBK_ERR_ARG); a barrier wait that expires gives MBK_ERR_TIMEOUT (the
 * workspace must then be re-bound).  The debug hook's skip_wg makes that
 * workgroup never arrive, to force the timeout from the host. */
int mbk_barrier_stress(mbk_model *m, int32_t n, void *stream, int32_t *first_bad);

/* Number of intervals (and ablation launches) per step: 5 per layer + 1.
 * Passage: the MegaBake article, "What I ran, on a CPU" (intervals per layer
 * after folding small producers into their consumers, plus the ones for the
 * embedding and the vocabulary head); here the embedding is folded too. */
int mbk_num_intervals(const mbk_model *m, int32_t *n);

/* Passage: none on the pages; a test hook of this repository.
 * Test hook: limit every bounded wait to `spin_limit` polls (0 = default,
 * 2^22) and make workgroup `skip_wg` (-1 = none) of the persistent kernel
 * leave at interval `skip_interval` without running it, so a test can force
 * the watchdog from the host: the waits of the workgroups that need its
 * results (or its barrier arrival) expire and the step reports
 * MBK_ERR_TIMEOUT through mbk_check. */
int mbk_set_debug(mbk_model *m, int32_t spin_limit, int32_t skip_wg, int32_t skip_interval);

/* Phase timer (the README's per-barrier-interval timer, section "Current
 * performance"): when buf != NULL, every workgroup of every following launch
 * writes the device wall clock (100 MHz) into buf as uint64
 * [interval][workgroup][4]: [0] interval start, [1] inputs loaded (written only by
 * workgroups with work in the interval), [2] body
 * done, [3] grid barrier passed (barrier mode only); entries of intervals
 * where a workgroup has no work are 0.  The stamps are stores issued during
 * the step (the timer takes no LDS).  buf must hold n_intervals * n_CUs * 32
 * bytes; NULL switches the timer off. */
int mbk_set_phase_trace(mbk_model *m, void *buf, size_t bytes);

/* Attention split policy: each split of the cached context covers at least
 * min_positions positions (default 128); contexts up to that length run
 * unsplit.  The number of splits is bounded by the plan (at most one per 32
 * cached positions, per workgroup of an item group's share of the device, and
 * as many as the 16 KiB merge scratch holds). */
int mbk_set_attention_split(mbk_model *m, int32_t min_positions);

/* Attention work items (the GQA packing of the flash-decoding step, README
 * mirror "Current status"): heads_per_item = 1 gives one item per (query head,
 * split); G = n_heads / n_kv_heads packs the G query heads of a KV head into
 * one item, so each cached key and value is read once; 0 (default) chooses one
 * query head per item unless there are more query heads than workgroups (on
 * MI355X the shorter per-item chain wins: the G readers of a KV head mostly
 * hit the caches).  Only before the schedule is planned (as
 * mbk_set_workgroups); MBK_ERR_ARG for any other value. */
int mbk_set_attention_items(mbk_model *m, int32_t heads_per_item);

/* Weight storage formats (mbk_set_weight_format). */
enum { MBK_WEIGHTS_BF16 = 0, MBK_WEIGHTS_FP8_E4M3 = 1 };

/* Stores the projection matrices and the vocabulary projection as 8-bit
 * codes instead of bf16, halving the weight bytes each decode step streams.
 * Passage: the project site, "Next" (FP8 among the directions the project
 * names); the format and scaling are this repository's readings: OCP 8-bit
 * floating point, E4M3 variant (bias 7, 3 mantissa bits, subnormals, largest
 * finite 448, no infinities), one power-of-two scale 2^e per output row (e the
 * smallest integer >= -126 with max|w| / 2^e <= 448, 0 for a zero row, so no
 * weight saturates), each code the weight divided by the scale (exactly)
 * rounded to nearest, ties to even, the sign of zero kept.  mbk_pack_weights
 * quantises the bf16 sources on the device; the embedding row gather keeps
 * the bf16 table and the vocabulary projection reads an fp8 copy of it; norm
 * weights and biases stay bf16; activations enter the dot products as fp32.
 * Only before the schedule is planned (as mbk_set_workgroups): MBK_ERR_STATE
 * after, MBK_ERR_ARG for an unknown format; planning fails with
 * MBK_ERR_UNSUPPORTED unless hidden, n_heads*head_dim and intermediate are
 * multiples of 16.  mbk_prefill on an fp8 handle runs the same quantised
 * model (each code widened exactly to bf16 in the GEMM, the row's scale
 * applied to its output). */
int mbk_set_weight_format(mbk_model *m, int32_t format);

/* Selects MBK_SYNC_DATAFLOW or MBK_SYNC_BARRIER for following steps
 * (the passages are given with the enum above).  MBK_ERR_ARG for any other
 * value. */
int mbk_set_sync_mode(mbk_model *m, int32_t mode);

/* How mbk_decode_step launches the persistent kernel.  Every workgroup of it
 * must be resident at once (they wait for one another).
 * PLAIN (default): an ordinary launch of one workgroup per compute unit,
 *   each workgroup taking most of its unit's LDS, so that an otherwise idle
 *   device holds all of them; the caller keeps other kernels off the device
 *   while a step runs (a workgroup kept out by another kernel only starts
 * *   when that kernel ends; the bounded waits report MBK_ERR_TIMEOUT if that
 *   takes too long).
 * COOPERATIVE: a cooperative launch, which the runtime admits only when all
 *   workgroups can be resident; about 15 us more per step on MI355X.
 * Passage: the MegaBake article, "How a model gets in", step 6 (the plan is
 * compiled into a single cooperative kernel); the plain launch is this
 * repository's choice.  MBK_ERR_ARG for any other value. */
enum { MBK_LAUNCH_PLAIN = 0, MBK_LAUNCH_COOPERATIVE = 1 };
int mbk_set_launch_mode(mbk_model *m, int32_t mode);

/* Passage: the MegaBake article, "What a megakernel is" (one resident block
 * per streaming multiprocessor working through a task list).
 * Number of workgroups of the persistent kernel (one per compute unit); n = 0
 * (default) uses every compute unit of the current device.  Only before the
 * schedule is planned (the first mbk_pack_weights / mbk_alloc_kv /
 * mbk_describe); a launch on a device with fewer compute units fails with
 * MBK_ERR_UNSUPPORTED.  With n > 0 the handle plans without touching a device. */
int mbk_set_workgroups(mbk_model *m, int32_t n);

/* Passage: none on the pages; this repository's introspection of its plan.
 * Plans the schedule if needed and writes a NUL-terminated JSON summary of it
 * (workgroups, threads, waves per role, intervals, packed/workspace/LDS/ring
 * bytes, task counts and sizes, attention splits and piece size) into buf.
 * MBK_ERR_SIZE if len is too small. */
int mbk_describe(mbk_model *m, char *buf, size_t len);

/* Message for the last non-zero status returned on this thread (valid
 * until the next failing call on the thread).  Passage: none on the pages;
 * the README mirror, "The compilation path", asks for errors rather than
 * silent fallbacks, and this carries their text. */
const char *mbk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MBK_H */
