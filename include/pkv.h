/*
 * pkv.h - paged KV decode attention on MI355X (gfx950): the C ABI.
 *
 * What it computes.  Exact single-token decode attention over a request's
 * whole paged key/value history (KV-cache engineering page, section "Costing
 * the bus before changing anything": each new token attends the entire
 * history).  The history is cut into tiles; each tile yields an output
 * already divided by its own softmax sum, plus the log-sum-exp of its
 * scores, and an FP32 merge weights tile t by exp(lse_t - max lse), adds
 * the weighted outputs, divides by the total weight and reports
 * max + log(total) as the merged log-sum-exp: the softmax of all the keys
 * at once (same page, section "Exact recent pages, compact older pages").
 *
 * Conventions for every entry point.
 *   - Return value: PKV_OK (0) or a negative PKV_ERR_* code.  No exception
 *     crosses the ABI.  pkv_last_error() gives a message for the calling
 *     thread that names the offending argument and the setting to change.
 *   - Validation is on the host and synchronous, before any device work.
 *     Kernels never check, never fault on a validated call and never sync.
 *   - Device pointers and streams belong to the caller.  The library never
 *     allocates device memory.  `stream` is a hipStream_t passed as void*
 *     (NULL = the default stream); every kernel of a call is queued on it
 *     in order and the host does not wait for it.
 *   - Handles (pool, stager, admission, live pool) hold host state without
 *     locks: calls on one handle from several threads must be serialized
 *     by the caller.  Calls on different handles are independent.
 *   - bf16 means IEEE binary32's upper 16 bits; all outputs are FP32.
 *   - The log-sum-exp is natural-log and includes the softmax scale:
 *     lse = log sum_j exp(scale * q.k_j).
 *
 * Arena layout (one device allocation shared by every layer; GPU memory
 * management page, "Pages held by right, borrowed or free").  Physical page
 * p holds page_tokens (64) consecutive tokens of one request, in every layer;
 * the arena is layer-major so that one layer's pages form one slab:
 *     arena[layer][page][K|V][kv_head][block]          (bf16)
 * A block is 64 tokens x 256 channels (32 KiB) stored as 2,048 pieces of
 * 16 bytes (8 bf16 values), in the order the decode kernel's wave loads
 * consume them, 64 pieces (1 KiB) per load instruction:
 *     K piece of token j, channels 8c..8c+7 is piece
 *         ((h*2 + t)*8 + c/4)*64 + (c%4)*16 + r,
 *         h = j/32, jj = j%32, t = (jj/4)%2, r = 4*(jj/8) + jj%4;
 *     V piece of channel d, tokens 8u..8u+7 is piece
 *         ((u/4)*16 + d/16)*64 + (u%4)*16 + d%16.
 * One (layer, page) is 2 * Hkv blocks (256 KiB at Hkv = 4), one physical
 * page num_layers times that, and a K+V token of one layer is
 * 2 * Hkv * 256 * 2 = 4,096 bytes at Hkv = 4 (GPU memory management page,
 * "A host pool that explains its own size").
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef PKV_H
#define PKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,      /* a null pointer, a negative size, an out-of-range index */
  PKV_ERR_AUTO_SIZE_REFUSED = -2, /* arena_bytes == 0: the pool size must be explicit */
  PKV_ERR_GEOMETRY = -3,         /* a head shape the kernels are not built for */
  PKV_ERR_WORKSPACE = -4,        /* workspace missing or smaller than pkv_decode_workspace_bytes */
  PKV_ERR_PAGE_TABLE = -5,       /* a page-table row the pool cannot serve */
  PKV_ERR_LAUNCH = -6,           /* the HIP runtime refused a launch */
  PKV_ERR_DEVICE = -7,           /* a HIP runtime call (copy, device query) failed */
  PKV_ERR_LEASE = -8,            /* a lease or live-pool step call out of order */
  PKV_ERR_BUSY = -9,             /* leases outstanding: retire before destroying */
  PKV_ERR_QUARANTINED = -10      /* a stager or live pool saw a failure: only retire
                                    (stager) or destroy (live pool) is accepted */
};

/* Geometry of the arena.  The kernels are built for head_dim = 256,
 * page_tokens = 64 and a query group (num_q_heads / num_kv_heads) of 1..16;
 * other shapes are refused with PKV_ERR_GEOMETRY. */
typedef struct pkv_geom {
  int32_t num_layers;    /* dense layers sharing the arena, >= 1            */
  int32_t num_kv_heads;  /* KV heads per layer, >= 1                        */
  int32_t head_dim;      /* channels per head: 256                          */
  int32_t page_tokens;   /* tokens per page: 64                             */
} pkv_geom;

typedef struct pkv_pool pkv_pool;   /* opaque host-side handle */

/* Message for the last failing call on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library ABI version (PKV_ABI_VERSION). */
#define PKV_ABI_VERSION 5
int32_t pkv_abi_version(void);

/* Bytes of one physical page (all layers) for `geom`. */
int pkv_page_bytes(const pkv_geom* geom, uint64_t* page_bytes_out);

/* ---------------------------------------------------------------- pool --
 * Wrap a caller-owned device arena of an explicit size as a page pool
 * (GPU memory management page, "A host pool that explains its own size":
 * an automatic size is refused outright).
 *   dev_arena    device pointer, 256-byte aligned, caller keeps it alive
 *                past pkv_pool_destroy.
 *   arena_bytes  explicit size: 0 -> PKV_ERR_AUTO_SIZE_REFUSED; it must be
 *                a whole number of pages (pkv_page_bytes), else
 *                PKV_ERR_INVALID_ARG with the nearest valid sizes named.
 * num_pages = arena_bytes / page_bytes.  Physical page ids are 0..num_pages-1.
 * The handle owns host memory only; pkv_pool_destroy frees it and never
 * waits on the device. */
int pkv_pool_create(const pkv_geom* geom, void* dev_arena, uint64_t arena_bytes,
                    pkv_pool** pool_out);
int pkv_pool_info(const pkv_pool* pool, int64_t* num_pages, uint64_t* page_bytes,
                  void** dev_arena);
int pkv_pool_destroy(pkv_pool* pool);

/* --------------------------------------------------------- compact pool --
 * Older pages kept in a compact representation (KV-cache engineering page,
 * section "Exact recent pages, compact older pages": a request's history is
 * served as runs of two representations; a page is converted only after
 * every layer has written all its tokens, then checksummed and published,
 * and is served exact before that).  The pages name no format; here:
 *   codes   E4M3 (OCP 8-bit float: sign, 4 exponent bits with bias 7,
 *           3 mantissa bits, largest finite 448), one byte per element;
 *   scale   one FP32 per (layer, page, K|V, kv head) block:
 *           amax / 448 in FP32 (1 for an all-zero block);
 *   code    E4M3 rounding of the FP32 quotient x / scale: to nearest, ties
 *           to even, saturating at 448, the input's sign kept; the element
 *           stands for value(code) * scale.  Inputs must be finite.
 * Arena layout: codes [layer][page][K|V][kv_head][16,384-byte block], then
 * scales [layer][page][K|V][kv_head] FP32.  A block holds 64 tokens x 256
 * channels as 1,024 pieces of 16 bytes in the compact kernel's load order:
 *   K piece ((h*2 + t)*4 + kk)*64 + q*16 + r: token 32h + 8(r/4) + 4t + r%4,
 *     bytes 0..7 channels 64kk + 8q .. +7, bytes 8..15 channels
 *     64kk + 32 + 8q .. +7;
 *   V piece (d/16)*64 + q*16 + d%16: channel d, bytes 0..7 tokens
 *     8q .. 8q+7, bytes 8..15 tokens 32 + 8q .. +7.
 * A compact page (all layers) is pkv_compact_page_bytes = num_layers x
 * 2 x num_kv_heads x (16,384 + 4) bytes: half an exact page plus scales.
 * A compact pool is created like an exact one (explicit size, whole pages)
 * and is accepted by pkv_page_table_validate/write and pkv_decode_attention
 * (default or MFMA kernel), which then reads codes and scales; it is refused
 * by pkv_append_kv and the stager (compact pages are immutable).
 * pkv_pool_format reports PKV_FORMAT_BF16 or PKV_FORMAT_E4M3. */
enum { PKV_FORMAT_BF16 = 0, PKV_FORMAT_E4M3 = 1 };
int pkv_compact_page_bytes(const pkv_geom* geom, uint64_t* page_bytes_out);
int pkv_compact_pool_create(const pkv_geom* geom, void* dev_arena, uint64_t arena_bytes,
                            pkv_pool** pool_out);
int pkv_pool_format(const pkv_pool* pool, int32_t* format_out);

/* Convert whole exact pages into compact pages and publish their CRC.
 * For i < n: exact page dev_src_pages[i] of `exact` (every layer, K and V,
 * every kv head) is written as compact page dev_dst_pages[i] of `compact`,
 * then dev_crc[i] receives the CRC-32 of that compact page.  Both pools must
 * have the same geometry.  dev_src_pages, dev_dst_pages: device int32 [n];
 * dev_crc: device uint32 [n].  An id outside its pool is skipped (nothing is
 * written, its CRC is 0); two entries naming one destination race.  The
 * caller converts a page only once all its tokens exist in every layer and
 * keeps serving it exact until it has the CRC and switches its tables
 * (publishes).
 * Queued on `stream` (two launches), no host wait; on a stream of its own it
 * runs beside decode, which never waits for it.
 *
 * CRC-32 here is the reflected 0x04C11DB7 code with initial value and final
 * xor 0xFFFFFFFF, over the compact page's bytes: for each layer in order,
 * its code blocks (2 x num_kv_heads x 16,384 bytes as stored), then its
 * scales (2 x num_kv_heads FP32, little endian).  pkv_compact_crc recomputes
 * it for compact pages already written (to verify a page before use). */
int pkv_compact_convert(const pkv_pool* exact, const pkv_pool* compact,
                        const int32_t* dev_src_pages, const int32_t* dev_dst_pages, int32_t n,
                        uint32_t* dev_crc, void* stream);
int pkv_compact_crc(const pkv_pool* compact, const int32_t* dev_pages, int32_t n,
                    uint32_t* dev_crc, void* stream);

/* ---------------------------------------------------------- page table --
 * A page table is int32 [batch][pt_stride] in row-major order: entry i of
 * row b is the physical page holding tokens [64 i, 64 i + 64) of request b.
 * ctx_lens is int32 [batch]: request b's history is tokens [0, ctx_lens[b]).
 * A row is served only if (checked here, on the host):
 *   - 0 <= ctx_lens[b] <= 64 * pt_stride;
 *   - its first ceil(ctx_lens[b] / 64) entries are pages in [0, num_pages);
 *     entry 0 is the request's attention-sink page, so a row with ctx > 0
 *     always names it (GPU memory management page, "Pages held by right,
 *     borrowed or free": the sink is always kept);
 *   - every later entry is -1 (padding is contiguous);
 *   - no physical page appears twice in the whole table.
 * pkv_page_table_validate only checks.  pkv_page_table_write checks, then
 * copies both host arrays to the caller's device arrays on `stream` and
 * waits for the stream to reach the end of that copy (so also for all work
 * queued on it before), so the host arrays may be any host memory and may be
 * reused on return: a set-up call.
 * pkv_page_table_write_async is the per-step form (the host never waits on
 * the step path: Staging without a stall, "Two copy queues and device-side
 * ordering"): it checks, queues both copies on `stream` in stream order
 * (after the decodes queued before it, which may still read dev_table) and,
 * if done_event (a hipEvent_t) is not NULL, records it after them; it
 * returns without waiting.  host_table and host_ctx_lens must be pinned host
 * memory (hipHostMalloc) that the caller leaves unchanged until done_event
 * has completed (e.g. a ring of such buffers, one per step in flight). */
int pkv_page_table_validate(const pkv_pool* pool, const int32_t* host_table,
                            const int32_t* host_ctx_lens, int32_t batch, int32_t pt_stride);
int pkv_page_table_write(const pkv_pool* pool, const int32_t* host_table,
                         const int32_t* host_ctx_lens, int32_t batch, int32_t pt_stride,
                         int32_t* dev_table, int32_t* dev_ctx_lens, void* stream);
int pkv_page_table_write_async(const pkv_pool* pool, const int32_t* host_table,
                               const int32_t* host_ctx_lens, int32_t batch, int32_t pt_stride,
                               int32_t* dev_table, int32_t* dev_ctx_lens, void* stream,
                               void* done_event);

/* -------------------------------------------------------------- decode --
 * Per-tile partials of decode attention for one layer.
 *
 * Tiles are tile_tokens long and start at logical token 0: tile t of
 * request b covers tokens [t T, min((t+1) T, ctx_b)).  One call covers the
 * token window [token_begin, token_begin + token_count); both are
 * multiples of tile_tokens, and the window writes slots
 * [token_begin / T, (token_begin + token_count) / T) of every row, each
 * shifted by opts.slot_offset.  With a compact pool the keys and values are
 * the compact pages' dequantised elements.  A tile
 * with no token of the request (ctx_b <= t T) is written as out = 0,
 * lse = -inf.  One call over the whole history (token_begin = 0) and
 * several calls over consecutive windows (staged tiles) write bit-identical
 * partials: the arithmetic of a tile depends only on the tile's own keys.
 *
 *   pool, layer      arena and layer 0..num_layers-1.
 *   q                device bf16 [batch][num_q_heads][head_dim] of this layer.
 *   dev_table        device int32 rows as above; entry i of a row is the
 *                    page of logical page (token_begin / 64 + i), so a
 *                    staged call may pass the full table offset by
 *                    token_begin / 64 entries, or a staging table.
 *                    pt_stride >= token_count / 64 is required.  An entry
 *                    outside [0, num_pages) is never dereferenced: its
 *                    tokens are skipped (validated tables have none).
 *   dev_ctx_lens     device int32 [batch], whole-history lengths.
 *   tile_tokens      multiple of 64.
 *   scale            softmax scale (1/sqrt(head_dim) for standard attention).
 *   part_out         device FP32 [batch][num_q_heads][num_slots][head_dim].
 *   part_lse         device FP32 [batch][num_q_heads][num_slots].
 *   workspace        device scratch of at least pkv_decode_workspace_bytes
 *                    (may be NULL when that is 0); contents need no init
 *                    and are dead after the stream reaches the call's end.
 *   opts             NULL for defaults (see pkv_decode_opts).
 */
typedef struct pkv_decode_opts {
  int32_t kernel;        /* 0 default, 1 VALU (fdot2 + FP32 FMA), 2 MFMA (16x16x32 bf16) */
  int32_t split_tokens;  /* 0 default; else tokens per work-group, a multiple of 64 dividing
                            tile_tokens, at most 16384 for the MFMA kernel and compact
                            pools (PKV_ERR_INVALID_ARG beyond).  The split is a pure function of these options and
                            tile_tokens, never of batch, lengths or the device, so staged and
                            resident calls with the same options agree bit for bit. */
  int32_t slot_offset;   /* 0 default; added to every slot the call writes, so the runs of
                            two representations (a compact older run and an exact recent
                            run, each with its own table) fill disjoint slots of one
                            partial buffer for a single merge. */
} pkv_decode_opts;

int pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                               int32_t token_count, int32_t tile_tokens,
                               const pkv_decode_opts* opts, uint64_t* bytes_out);

int pkv_decode_attention(const pkv_pool* pool, int32_t layer, const void* q,
                         const int32_t* dev_table, int32_t pt_stride,
                         const int32_t* dev_ctx_lens, int32_t batch, int32_t num_q_heads,
                         int32_t token_begin, int32_t token_count, int32_t tile_tokens,
                         float scale, float* part_out, float* part_lse, int32_t num_slots,
                         void* workspace, uint64_t workspace_bytes,
                         const pkv_decode_opts* opts, void* stream);

/* Decode and merge of a whole history in one call: the tile partials exactly
 * as pkv_decode_attention with token_begin = 0, then out [batch][num_q_heads]
 * [head_dim] and lse [batch][num_q_heads] exactly as pkv_merge_partials over
 * all num_slots slots, bit for bit (the same FP32 merge runs in both).  The
 * call must write every slot: token_count / tile_tokens == num_slots and
 * opts.slot_offset == 0.  Where a tile holds several splits and a row has at
 * most 64 splits, the tile finalize and the final merge are one launch (one
 * kernel boundary fewer per layer than decode + merge).  out: FP32 device,
 * 16-byte aligned; lse: FP32 device.  Other arguments and errors as
 * pkv_decode_attention. */
int pkv_decode_attention_merged(const pkv_pool* pool, int32_t layer, const void* q,
                                const int32_t* dev_table, int32_t pt_stride,
                                const int32_t* dev_ctx_lens, int32_t batch, int32_t num_q_heads,
                                int32_t token_count, int32_t tile_tokens, float scale,
                                float* part_out, float* part_lse, int32_t num_slots, float* out,
                                float* lse, void* workspace, uint64_t workspace_bytes,
                                const pkv_decode_opts* opts, void* stream);

/* The same call for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Identical to pkv_decode_attention_merged (same kernels, same bits) except
 * that the split partials of a tile with several splits live in a static
 * device buffer of the library, PKV_STATIC_SCRATCH_BYTES (16 MiB) per GPU,
 * which the library holds from its first use on that GPU until the process
 * ends, instead of a caller workspace.  The call itself allocates nothing
 * (no hipMalloc, no allocating library routine).  A call needing more than
 * that (pkv_decode_workspace_bytes) is refused with PKV_ERR_WORKSPACE; one
 * needing none (opts.split_tokens = tile_tokens, or the default split equal
 * to the tile) never touches the buffer.  Every call on one GPU shares the
 * buffer and finds the last call's contents in it (nothing in it needs a
 * start value): two calls that may run at the same time on one GPU (on
 * different streams, or from different threads) race, so order them on one
 * stream.  Other arguments, outputs and errors as
 * pkv_decode_attention_merged. */
#define PKV_STATIC_SCRATCH_BYTES (16ull << 20)
int pkv_decode_attention_merged_noalloc(const pkv_pool* pool, int32_t layer, const void* q,
                                        const int32_t* dev_table, int32_t pt_stride,
                                        const int32_t* dev_ctx_lens, int32_t batch,
                                        int32_t num_q_heads, int32_t token_count,
                                        int32_t tile_tokens, float scale, float* part_out,
                                        float* part_lse, int32_t num_slots, float* out,
                                        float* lse, const pkv_decode_opts* opts, void* stream);

/* ---------------------------------------------------- runs in one launch --
 * The runs of two representations (KV-cache engineering, section "Exact
 * recent pages, compact older pages": a compact older run and an exact
 * recent run, each with its own pages) decoded by one launch: every run's
 * tiles are exactly the partials pkv_decode_attention writes for that run
 * alone (token_begin 0, one work-group per tile, opts.slot_offset =
 * slot_offset), bit for bit, but the runs' work-groups share one grid, so
 * neither run waits for the other's last work-group and the launch has one
 * ramp and one drain.  Then pkv_merge_partials over all slots, as for
 * separate calls.
 *   runs[k].pool           bf16 or compact (E4M3) pool; every run's pool has
 *                          the same KV heads, and layer is valid in each.
 *   runs[k].dev_table,     the run's own rows (entry i = page i of the run)
 *   pt_stride, dev_ctx_lens  and lengths, device int32.
 *   runs[k].token_count    a multiple of tile_tokens, pt_stride * 64 or less.
 *   runs[k].tile_tokens    multiple of 64 in 64..16384 (a tile is one
 *                          work-group's split).
 *   runs[k].slot_offset    first slot of the run; the runs' slot ranges
 *                          must not overlap and must fit num_slots.
 * n_runs 1 or 2; the query group must be one the MFMA kernel is built for
 * (1..8, 12, 16).  Other arguments as pkv_decode_attention. */
typedef struct pkv_decode_run {
  const pkv_pool* pool;
  const int32_t* dev_table;
  int32_t pt_stride;
  const int32_t* dev_ctx_lens;
  int32_t token_count;
  int32_t tile_tokens;
  int32_t slot_offset;
} pkv_decode_run;

int pkv_decode_attention_runs(int32_t layer, const void* q, int32_t batch, int32_t num_q_heads,
                              const pkv_decode_run* runs, int32_t n_runs, float scale,
                              float* part_out, float* part_lse, int32_t num_slots, void* stream);

/* ------------------------------------------------ per-request tiles --
 * Tiles of their own length for each request of a batch (the same per-tile
 * partials and merge as above; the KV-cache engineering page, section
 * "Exact recent pages, compact older pages", leaves the tile length free).
 * A batch of very different lengths cut into one tile length leaves most
 * work-groups short or idle; planning each request's tiles so that every
 * work-group of the launch carries about the same number of tokens fills
 * the GPU evenly.  The plan depends on all the batch's lengths, so a
 * request's partials (not its merged result, up to rounding) depend on the
 * batch: use the fixed tiling above where bit-identity across batches or
 * staged windows matters.
 *
 * pkv_plan_tiles (host only): tau = the smallest multiple of 64 up to
 * max_tile_tokens for which num_kv_heads * sum_b ceil(ctx_b / tau) <=
 * work_groups (max_tile_tokens if none); request b is cut into n_b =
 * ceil(ctx_b / tau) tiles of host_row_tile_tokens[b] = ctx_b / n_b rounded
 * up to a multiple of 64 (64 for an empty request); *max_tiles_out =
 * max(1, max_b n_b).  Deterministic.
 *   host_ctx_lens [batch] >= 0; work_groups >= 1 (256 = one per CU on
 *   MI355X); max_tile_tokens a multiple of 64 in 64..16384.
 *
 * pkv_decode_attention_rows: tile t of request b covers tokens
 * [t T_b, min((t+1) T_b, ctx_b)) with T_b = dev_row_tile_tokens[b]; tiles
 * 0 .. max_tiles-1 of every row are written to slots opts.slot_offset + t
 * (out = 0, lse = -inf for a tile past ctx_b).  max_row_tile_tokens >=
 * every T_b (the plan's maximum); pt_stride >= max_tiles *
 * max_row_tile_tokens / 64.  MFMA kernel and bf16 pools only
 * (opts.kernel 0 or 2, opts.split_tokens 0); no workspace (each tile is one
 * work-group).  A device T_b that is not a multiple of 64 in 64..16384, or
 * a request longer than max_tiles * T_b, is not silently cut: the affected
 * row's partial carries lse = NaN (the host cannot read device lengths
 * without a sync).  Other arguments as pkv_decode_attention. */
int pkv_plan_tiles(const int32_t* host_ctx_lens, int32_t batch, int32_t num_kv_heads,
                   int32_t work_groups, int32_t max_tile_tokens, int32_t* host_row_tile_tokens,
                   int32_t* max_tiles_out);
int pkv_decode_attention_rows(const pkv_pool* pool, int32_t layer, const void* q,
                              const int32_t* dev_table, int32_t pt_stride,
                              const int32_t* dev_ctx_lens, int32_t batch, int32_t num_q_heads,
                              const int32_t* dev_row_tile_tokens, int32_t max_row_tile_tokens,
                              int32_t max_tiles, float scale, float* part_out, float* part_lse,
                              int32_t num_slots, const pkv_decode_opts* opts, void* stream);

/* --------------------------------------------------------------- merge --
 * FP32 log-sum-exp merge of the partials of each row (KV-cache engineering
 * page, section "Exact recent pages, compact older pages").  For row r,
 * with M = max_t lse[r][t]:
 *   M = -inf (every slot empty) -> out[r] = 0, lse[r] = -inf;
 *   else w_t = exp(lse[r][t] - M), W = sum_t w_t,
 *        out[r] = sum_t w_t part_out[r][t] / W, lse[r] = M + log W.
 * Slots with lse = -inf add nothing (their part_out is never read into the
 * sums), and the sums run over t in increasing order, so inserting empty
 * slots leaves the result bit-identical and a single slot merges to itself.
 * A slot with lse = NaN (a flagged partial) makes its row's out and lse NaN.
 *   part_out [rows][num_slots][head_dim], part_lse [rows][num_slots] (rows =
 *   batch * num_q_heads), out [rows][head_dim], lse [rows]; all FP32 device.
 * head_dim must be 256.  num_slots >= 1. */
int pkv_merge_partials(const float* part_out, const float* part_lse, int32_t rows,
                       int32_t num_slots, int32_t head_dim, float* out, float* lse,
                       void* stream);

/* -------------------------------------------------------------- append --
 * Write the new token of each request into its page of one layer, in the
 * block layout above, so the next decode step attends over it (GPU memory
 * management page, "Pages held by right, borrowed or free": the newest
 * pages stay on the device).
 *   dev_table      device int32 [batch][pt_stride], rows as for decode
 *                  (entry i = logical page i of the request).
 *   dev_positions  device int32 [batch]: the token index to write, normally
 *                  the old length (the caller then passes length + 1 to
 *                  decode), counted from the first logical page of the row
 *                  (with a lease's staging table: minus window_begin); -1
 *                  skips a request.  A position whose page entry
 *                  lies outside the row or outside [0, num_pages) is not
 *                  written (never dereferenced); validated tables have none.
 *   k_new, v_new   device bf16 [batch][num_kv_heads][256], 16-byte aligned.
 * Only the 16-byte K pieces and 2-byte V elements of that token change; the
 * rest of the page is untouched.  Queued on `stream`, no host wait. */
int pkv_append_kv(const pkv_pool* pool, int32_t layer, const int32_t* dev_table,
                  int32_t pt_stride, const int32_t* dev_positions, int32_t batch,
                  const void* k_new, const void* v_new, void* stream);

/* ---------------------------------------------------------- staged tiles --
 * History held in pinned host memory, brought to the device one window of
 * one layer at a time under a lease (Staging without a stall, sections "Two
 * copy queues and device-side ordering" and "Leases instead of buffers";
 * KV-cache engineering, "Staging layers under a lease"; GPU memory
 * management, "Staging as a lease").
 *
 * The host arena has the layout of a pool with `host_layers` layers and the
 * staging pool's head shape: host[layer][page][K|V][kv_head][block].  With
 * a compact staging pool it has the compact layout instead (codes of every
 * layer, then their scales) and each window's scales are copied with its
 * codes; compact pages are immutable, so a seal with write_back_tail is
 * refused.  The
 * stager owns `num_buffers` staging buffers in layer 0 of the staging pool,
 * each of max_batch x window_tokens/64 pages, and three caller streams:
 *   copy       host -> device window copies;
 *   compute    the caller's work on a lease (decode, append) runs here;
 *   writeback  device -> host write-back of changed tail rows.
 * Ordering is on the device: a window's copy waits for the previous readers
 * of the buffer it overwrites (that lease's consumer and write-back events)
 * and, when it reads a host page that received a tail row since the last
 * retire, for the latest write-back; the compute stream waits for the copy,
 * and the write-back waits for the compute stream's consumer event.  Only
 * pkv_stager_retire blocks the host.
 * Each window's copy is split in two: the first half on `copy`, the second
 * on a stream the stager creates and owns (default priority, destroyed with
 * the stager), so one copy's wait overlaps the other's transfer.
 *
 * Lifecycle.  pkv_lease_begin queues the copy of tokens
 * [window_begin, window_begin + window_tokens) of every request (runs of
 * consecutive host pages in one copy each) and fills *lease: the staging
 * table (entry i of row b = logical page window_begin/64 + i) to pass to
 * pkv_decode_attention / pkv_append_kv with the staging pool and
 * lease.staging_layer, on the compute stream.  pkv_lease_seal records the
 * consumer event after that work and, if write_back_tail, writes back the
 * changed tail rows only: the K and V of each request's last token
 * (ctx_lens[b] - 1) when it lies in the window, 2 x num_kv_heads x 256 bf16
 * per request (4,096 bytes at 4 KV heads), stored into the host page by a
 * kernel on the write-back stream (GPU memory management page, "Staging as
 * a lease").  For a bf16 staging pool the host arena must be pinned memory
 * the device can address (hipHostMalloc); create fails otherwise.  A lease
 * is refused while the previous one is still unsealed; a seal must name
 * the open lease.  Stage generations only increase.
 * pkv_stager_retire waits for every sealed lease and returns their count as
 * receipts.  Any HIP failure quarantines the stager: begin and seal are
 * refused, retire drains the copy, write-back and compute streams and the
 * device, and if a drain fails everything stays retained.  Destroy never
 * waits: with leases outstanding it refuses (PKV_ERR_BUSY).
 * dev_tables is device int32 [num_buffers][max_batch][window_tokens/64],
 * written once by create.  The host arena and staging pool must outlive the
 * stager. */
typedef struct pkv_stager pkv_stager;
typedef struct pkv_lease {
  uint64_t generation;      /* stage generation, 1, 2, ... per stager          */
  int32_t layer;            /* host layer staged                               */
  int32_t window_begin;     /* first token of the window                       */
  int32_t buffer;           /* staging buffer used                             */
  int32_t staging_layer;    /* layer of the staging pool to decode from (0)    */
  const int32_t* dev_table; /* staging page table, rows of pt_stride entries   */
  int32_t pt_stride;        /* window_tokens / 64                              */
} pkv_lease;

int pkv_stager_create(const pkv_pool* staging, void* host_arena, uint64_t host_bytes,
                      int32_t host_layers, int32_t max_batch, int32_t window_tokens,
                      int32_t num_buffers, int32_t* dev_tables, void* copy_stream,
                      void* compute_stream, void* writeback_stream, pkv_stager** out);
int pkv_lease_begin(pkv_stager* stager, int32_t layer, const int32_t* host_table,
                    int32_t pt_stride, const int32_t* host_ctx_lens, int32_t batch,
                    int32_t window_begin, pkv_lease* lease);
int pkv_lease_seal(pkv_stager* stager, const pkv_lease* lease, int32_t write_back_tail);
int pkv_stager_retire(pkv_stager* stager, int64_t* receipts);
int pkv_stager_info(const pkv_stager* stager, uint64_t* generation, int64_t* unretired,
                    int32_t* open, int32_t* quarantined);
/* Mark the transport failed from the caller's side (its own work on a lease
 * failed): the stager is quarantined exactly as after a HIP failure. */
int pkv_stager_fail(pkv_stager* stager);
int pkv_stager_destroy(pkv_stager* stager);

/* ------------------------------------------------------------ admission --
 * Which logical pages of which contexts hold device pages, decided at step
 * boundaries by explicit arithmetic (Staging without a stall, section
 * "Admission that does arithmetic"; GPU memory management, section "Pages
 * held by right, borrowed or free").  Host only: no device memory is touched
 * and no HIP call is made.  Device page ids are 0..num_pages-1 of a pool of
 * that explicit size (0 is refused).
 *
 * A context holds its sink page (logical page 0) and its newest pages:
 * `target` pages by right plus up to `burst` borrowed while pages are free;
 * its floor is the sink plus one page.  pkv_admit_step takes the contexts
 * active in this step, in priority order, with their lengths in tokens, and
 * for each fills the sink and then the newest pages downward.  A missing
 * page comes from, in order: (1) the context's own page outside its window,
 * (2) a free page (marked borrowed once the context holds its target),
 * (3) while below target, other contexts least recently active first: their
 * borrowed pages, then pages above their target, then whole idle contexts,
 * (4) the context's own oldest non-sink page older than the one wanted.  If
 * none exists the context is refused for the step when it lacks its sink or
 * floor; otherwise its window stays shorter and the rest is staged.
 *   table   int32 [n][pt_stride] out: device page of each logical page, -1
 *           where the page is not resident (to be staged from the host).
 *   status  int32 [n] out: PKV_ADMIT_FULL, PKV_ADMIT_PARTIAL or
 *           PKV_ADMIT_REFUSED_STEP.
 * Every fill and reclamation is counted (pkv_admit_get_counts) and logged
 * (pkv_admit_events drains the log; it grows until drained). */
enum {
  PKV_ADMIT_REUSE_OWN = 1, PKV_ADMIT_TAKE_FREE = 2, PKV_ADMIT_RECLAIM_BORROWED = 3,
  PKV_ADMIT_RECLAIM_ABOVE_TARGET = 4, PKV_ADMIT_RECLAIM_IDLE = 5, PKV_ADMIT_SHRINK_OWN = 6,
  PKV_ADMIT_REFUSED = 7
};
enum { PKV_ADMIT_FULL = 0, PKV_ADMIT_PARTIAL = 1, PKV_ADMIT_REFUSED_STEP = 2 };
typedef struct pkv_admit pkv_admit;
typedef struct pkv_admit_counts {
  int64_t steps, reuse_own, take_free, reclaim_borrowed, reclaim_above_target, reclaim_idle,
      shrink_own, refused, free_pages;
} pkv_admit_counts;
typedef struct pkv_admit_event {
  int64_t step;      /* step number (1, 2, ...)                                  */
  int32_t kind;      /* PKV_ADMIT_REUSE_OWN .. PKV_ADMIT_REFUSED                 */
  int32_t context;   /* the context served (or refused)                          */
  int32_t victim;    /* context the page came from; -1 for the free list        */
  int32_t page;      /* device page; -1 for a whole-context eviction or refusal */
  int32_t logical;   /* logical page it now holds; -1 if none                    */
} pkv_admit_event;
int pkv_admit_create(int64_t num_pages, int32_t page_tokens, pkv_admit** out);
int pkv_admit_add(pkv_admit* a, int32_t ctx, int32_t target_pages, int32_t burst_pages);
int pkv_admit_set_target(pkv_admit* a, int32_t ctx, int32_t target_pages, int32_t burst_pages);
int pkv_admit_remove(pkv_admit* a, int32_t ctx);
int pkv_admit_step(pkv_admit* a, int32_t n, const int32_t* ctx_ids, const int64_t* lengths,
                   int32_t* table, int32_t pt_stride, int32_t* status);
int pkv_admit_get_counts(const pkv_admit* a, pkv_admit_counts* out);
int pkv_admit_events(pkv_admit* a, pkv_admit_event* out, int32_t cap, int32_t* n_out);
int pkv_admit_destroy(pkv_admit* a);

/* ------------------------------------------------------------ live pool --
 * Decode steps over histories whose authoritative copy is in pinned host
 * memory, with a device pool smaller than the histories (Staging without a
 * stall, sections "Admission that does arithmetic", "Two copy queues and
 * device-side ordering" and "Leases instead of buffers"; GPU memory
 * management, sections "Pages held by right, borrowed or free" and "Staging
 * as a lease").  Each step the admission planner above (the runtime owns
 * one, over the pool's pages) decides which logical pages of each context
 * hold pool pages: the sink and the newest pages.  A pool page that turns
 * hot (it now serves a (context, logical page) whose bytes it does not
 * hold) is copied in from the host once; every other logical page of the
 * history is staged, one layer at a time, into the staging pool.  One
 * decode launch per layer reads both through a composed table, so a step's
 * partials, out and lse are bit-identical to pkv_decode_attention_merged of
 * a fully resident copy of the same histories at the same tile_tokens and
 * split (a tile's arithmetic depends only on its logical tokens).  The new
 * token is appended on the device and only its rows are written back to the
 * host pages (2 x num_kv_heads x 256 bf16 per context and layer).
 *
 * The composed table (device int32, inside dev_state): entry i of row b is
 * the pool page of logical page i if resident, else num_pages(pool) + s for
 * staging page s; -1 past the history.
 *
 * pkv_live_create
 *   pool        bf16 pool of L layers whose pages admission hands out.
 *   stage       bf16 pool, same KV heads; its num_layers K is the number of
 *               staging buffers (layer l stages into its layer l % K) and
 *               its num_pages the most pages one step may stage (a step that
 *               stages more fails and quarantines the runtime).
 *   host_arena  pinned host memory the device can address (hipHostMalloc),
 *               the layout of an L-layer pool: host[layer][page][K|V]
 *               [kv_head][block]; host_bytes a whole number of such pages.
 *   max_batch   contexts per step, at most; pt_stride: pages per table row.
 *   dev_state   device int32 [max_batch * (pt_stride + 2)], the caller's:
 *               the step's composed table, lengths and append positions.
 *   streams     copy (host -> device pages), compute (table copy, append,
 *               decode, merge) and write-back (new rows -> host), the
 *               caller's, default priority.  Every run of pages is copied as
 *               two halves, one on the copy stream and one on a second copy
 *               stream the runtime creates and owns (default priority).
 *   The runtime allocates a pinned ring of 4 step tables (host memory, at
 *   create) and never device memory.
 * pkv_live_add / pkv_live_set_target / pkv_live_remove: contexts, with the
 *   target / burst / floor of pkv_admit_*.  pkv_live_admission gives the
 *   runtime's planner for pkv_admit_get_counts / pkv_admit_events only.
 * pkv_live_step_begin: n contexts (priority order) with their lengths in
 *   tokens including this step's new token, and host_rows [n][host_stride]:
 *   the host page of each logical page.  Fills status [n] (PKV_ADMIT_FULL,
 *   _PARTIAL, _REFUSED_STEP; a refused context decodes nothing, out 0 and
 *   lse -inf, and is not appended) and *info (may be NULL).  Runs admission,
 *   composes the table and queues its copy on the compute stream; waits on
 *   the host only when the ring is full (the GPU 4 steps behind).  A step
 *   is open from its begin until its last layer is queued: meanwhile a new
 *   begin and pkv_live_remove are refused with PKV_ERR_LEASE.  A context
 *   removed and added again under the same id takes none of its old pages'
 *   bytes (its pages are copied in afresh).
 * pkv_live_layer: one layer of the open step, each layer once.  On the copy
 *   stream, after the previous step's write-back of this layer and the last
 *   reader of the staging buffer: the hot pages' and staged pages' slices
 *   of this layer.  On the compute stream: k_new / v_new ([n][Hkv][256]
 *   bf16, 16-byte aligned) appended at position length - 1, then
 *   pkv_decode_attention_merged over the composed table with token_count =
 *   num_slots x tile_tokens (every length must fit) into part_out,
 *   part_lse, out, lse ([n][num_q_heads]...).  On the write-back stream,
 *   after the decode: the new rows into the host pages.  Arguments are
 *   checked before anything is queued.
 * pkv_live_destroy waits for the three streams, then frees host state.  A
 *   HIP failure quarantines the runtime: every call but destroy is refused.
 *
 * Compact older pages in the live pool (KV-cache engineering, sections
 * "Exact recent pages, compact older pages" and "What the hybrid tier
 * buys": with the history in host memory the bus sets the pace, so a
 * representation pays for itself by the bus bytes per token it saves).
 * pkv_live_attach_compact (between steps, once)
 *   cstage        compact (E4M3) pool, same KV heads: its num_layers C is the
 *                 number of compact staging buffers (layer l uses buffer
 *                 l % C), its num_pages the most compact pages one step may
 *                 stage (more fails and quarantines the runtime).
 *   compact_host  pinned host memory holding the compact copy of every host
 *                 page in the layout of a compact pool of host_pages pages
 *                 and L layers (codes [layer][page], then scales
 *                 [layer][page]); compact_host_bytes exactly that size.
 *   compact_tile_tokens  tile of the compact run: a multiple of 64 in
 *                 64..16384 dividing pt_stride x 64.
 *   dev_cstate    device int32 [max_batch * (pt_stride + 1)], the caller's:
 *                 the compact run's table and lengths.
 * pkv_live_publish / pkv_live_retract (host page ids): mark host pages
 *   whose compact copy in compact_host is written (the caller converts a
 *   page once it is full in every layer, e.g. with pkv_compact_convert from
 *   its pool page while it is the resident tail, and publishes it), or no
 *   longer valid.  They take effect at the next pkv_live_step_begin.  The
 *   caller must not rewrite a page's compact bytes while a queued step may
 *   still copy them (until the copy stream has passed that step's layers).
 * With compact pages attached, pkv_live_step_begin stages a page that is
 *   not resident, full (all 64 tokens inside the length) and published as
 *   compact: its entry in the composed table is -1 (the exact run masks
 *   it), and it joins the request's compact run, in logical order, read
 *   from a compact staging page.  Every other page is served as before.
 *   info->compact_staged_pages counts them.  pkv_live_layer then copies the
 *   compact pages' codes and scales of the layer after the last reader of
 *   the buffer, and decodes both runs in one launch
 *   (pkv_decode_attention_runs): the exact run over the composed table with
 *   tiles of tile_tokens (opts.split_tokens 0 or tile_tokens; the other
 *   options are ignored) into slots 0 .. E-1, E = pt_stride x 64 /
 *   tile_tokens, the compact run into slots E .. E+C'-1, C' = pt_stride x
 *   64 / compact_tile_tokens; num_slots must be E + C'.  Then
 *   pkv_merge_partials into out and lse; workspace is unused.  The result
 *   is bit-identical to pkv_decode_attention_runs + pkv_merge_partials over
 *   resident copies of both runs.
 */
typedef struct pkv_live pkv_live;
typedef struct pkv_live_info {
  int64_t copied_in_pages;  /* pool pages filled from the host this step (every layer) */
  int64_t staged_pages;     /* pages staged for each layer this step */
  int32_t refused;          /* contexts refused this step */
  int32_t resident_pages;   /* pool pages the step reads */
  int64_t compact_staged_pages;  /* pages staged as compact for each layer this step */
} pkv_live_info;
int pkv_live_create(const pkv_pool* pool, const pkv_pool* stage, void* host_arena,
                    uint64_t host_bytes, int32_t max_batch, int32_t pt_stride, int32_t* dev_state,
                    void* copy_stream, void* compute_stream, void* writeback_stream,
                    pkv_live** out);
int pkv_live_add(pkv_live* live, int32_t ctx, int32_t target_pages, int32_t burst_pages);
int pkv_live_set_target(pkv_live* live, int32_t ctx, int32_t target_pages, int32_t burst_pages);
int pkv_live_remove(pkv_live* live, int32_t ctx);
int pkv_live_admission(pkv_live* live, pkv_admit** out);
int pkv_live_step_begin(pkv_live* live, int32_t n, const int32_t* ctx_ids, const int64_t* lengths,
                        const int32_t* host_rows, int32_t host_stride, int32_t* status,
                        pkv_live_info* info);
int pkv_live_layer(pkv_live* live, int32_t layer, const void* q, const void* k_new,
                   const void* v_new, int32_t num_q_heads, int32_t tile_tokens, float scale,
                   float* part_out, float* part_lse, int32_t num_slots, float* out, float* lse,
                   void* workspace, uint64_t workspace_bytes, const pkv_decode_opts* opts);
int pkv_live_attach_compact(pkv_live* live, const pkv_pool* cstage, void* compact_host,
                            uint64_t compact_host_bytes, int32_t compact_tile_tokens,
                            int32_t* dev_cstate);
int pkv_live_publish(pkv_live* live, const int32_t* host_pages, int32_t n);
int pkv_live_retract(pkv_live* live, const int32_t* host_pages, int32_t n);
int pkv_live_destroy(pkv_live* live);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
