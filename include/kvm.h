/*
 * kvm.h -- libkvmove: layerwise movement of KV-cache blocks between the paged
 * HBM layout and the persistent cross-layer Full Block layout, on one
 * AMD Instinct MI355X (gfx950).
 *
 * Four operations, each stream-ordered on the caller's stream:
 *   kvm_pack_full     paged pool  -> Full Block [T][L][C_KV]       (all layers)
 *   kvm_unpack_layer  Full Block layer slice -> paged slots          (one layer)
 *   kvm_merge_layer   hit rows || miss rows -> complete_layer        (one layer)
 *   kvm_batch_copy    many (src_off, dst_off, nbytes) objects        (one list)
 * and kvm_unpack_merge_layer, unpack and merge of one layer in one pass.
 *
 * Sources (page title, section):
 *   DualPath KV Loading, "Dual-Path Loading", key-objects table: the persisted
 *     Full Block is a [T_hit, L, C_KV] view; hit_layer[l] is its layer-l slice
 *     [T_hit, C_KV]; miss_layer[l] is [T_miss, C_KV]; complete_layer[l] is
 *     [T_all, C_KV], the hit rows followed by the miss rows.
 *   DualPath KV Loading, "two read paths": per layer the hit slice is written
 *     into an HBM layer slot, and hit and miss are concatenated by token.
 *   DualPath KV Loading, design checklist: the Full Block <-> layer-block
 *     conversion keeps token, layer and KV-head order.
 *   Tutti reading notes, prerequisites 3 (eq. 2): paged blocks of B_tokens
 *     tokens, not contiguous, linked by a block table.
 *   Tutti reading notes, prerequisites 5 (eq. 3-4) and design 1: one K and one
 *     V object per layer per block; one compact (address, length) entry per
 *     contiguous object; one launch per layer rather than one call per object
 *     ("pseudo-code 1", layer-level batched retrieval).
 *   Mooncake Ascend Transports, "why addresses need relocation": a transfer is
 *     named by offsets from a known base, not by raw foreign pointers; and
 *     "back to the real objects": an enqueued copy is not a finished copy.
 *
 * Conventions for every call
 *   - Device pointers are HIP device addresses on the context's device. A Full
 *     Block, miss rows or complete_layer may also live in pinned host memory
 *     (hipHostMalloc): the kernels then read or write it over PCIe through its
 *     device-visible address (DualPath's host-DRAM prompt buffers). So may a
 *     batched copy's source or destination buffer (a restore from a host-DRAM
 *     staging buffer); its descriptor array stays in device memory. Host
 *     arrays (kvm_seq, kvm_merge_seq) are read during the call and may be
 *     reused as soon as it returns: their contents travel to the kernels as
 *     kernel arguments, up to 128 records per launch.
 *   - The caller owns every buffer and stream and keeps device buffers alive
 *     until the stream has run the work. The library keeps no caller pointer
 *     after a call returns.
 *   - All operations are asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL is the null stream). KVM_OK means "enqueued"; the result is
 *     there once the stream (or an event recorded after the call) completes.
 *   - Every argument is validated before anything is enqueued: a call that
 *     returns KVM_EINVAL or KVM_ERANGE has enqueued nothing. One that returns
 *     KVM_ENOMEM has written no caller buffer (only the library's own scratch
 *     may have been). A KVM_EHIP from a failed launch can leave the call's
 *     earlier launches (its first records) enqueued.
 *   - Payload is opaque bytes: no value is converted, so bf16 NaN payloads,
 *     -0 and denormals move bit for bit.
 *   - Any byte alignment is accepted. Pointers, strides and row sizes that are
 *     all multiples of 16 bytes take 16-byte vector moves; otherwise the widest
 *     unit dividing all of them is used.
 *   - Device-side guards: a block-table entry outside [0, num_blocks) or a copy
 *     object outside its buffer is skipped (its destination is left as it was)
 *     and counted; kvm_take_device_errors() returns the count.
 *   - One context per host thread; calls on one context are not thread-safe.
 *     One context may be used on several streams: the calls order their use
 *     of the context's scratch across streams themselves (see kvm_unpack_layer
 *     and kvm_batch_copy).
 *   - Waits. No pack, unpack, merge, fused or batched-copy call waits for the
 *     whole device. Where one would need a buffer that launches already
 *     enqueued may still read (its scratch grows; a second stream appears),
 *     it takes a new buffer and keeps the old one allocated until the next
 *     call that synchronises the device anyway: kvm_ctx_reserve (when it
 *     resizes or has such buffers to free), kvm_ctx_reserve_unpack,
 *     kvm_take_device_errors and kvm_destroy, the only calls that do. The
 *     host waits that remain are on events the library itself recorded, and
 *     only once a context has seen two streams (a replaced tile order waits
 *     for the launches that read it), plus kvm_ctx_set_checks' debug mode,
 *     which synchronises the call's own stream.
 *   - HIP graph capture: kvm_pack_full and kvm_merge_layer may be captured.
 *     They read no state the context keeps between calls (their records
 *     travel as kernel arguments), allocate nothing, record no event and
 *     clear nothing with a memset, so a replay moves the bytes the buffers
 *     hold then, through the pointers and sizes given at capture. Unpack and
 *     the fused call may not: their launches read the context's cached tile
 *     order, which a later call with other block tables may overwrite before
 *     the graph replays. kvm_batch_copy may not (its scratch and piece counts
 *     are the context's); kvm_batch_copy_noalloc may (see there).
 *   - Caller preconditions: the block tables of one unpack or fused call
 *     hold no repeated entry; pool rows described by the layout do not overlap;
 *     copy destinations are pairwise disjoint and do not overlap the sources.
 *     Violations give an unspecified (but in-bounds) result. The kernels do
 *     not check them; kvm_ctx_set_checks turns on host-side checks of the
 *     first and the last (a debug mode).
 */
#ifndef KVM_H
#define KVM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVM_ABI_VERSION 1

/* Status codes. */
#define KVM_OK 0
#define KVM_EINVAL (-1) /* null pointer, negative size or stride, malformed layout */
#define KVM_ERANGE (-2) /* layer outside [0, L), a size above a supported limit   */
#define KVM_ENOMEM (-3) /* device or pinned host memory could not be obtained      */
#define KVM_EHIP (-4)   /* a HIP runtime call or launch failed; see kvm_ctx_last_error */
#define KVM_ECHECK (-5) /* checks on (kvm_ctx_set_checks): a caller precondition is
                           violated; see kvm_ctx_last_error */

typedef struct kvm_ctx kvm_ctx;

/* Paged pool geometry (Tutti reading notes, prerequisites 3, eq. 2; one K and one
 * V object per layer per block, prerequisites 5). The token row of
 * (layer l, side s, block n, row r) starts at byte
 *     l*layer_stride + s*side_stride + n*block_stride + r*row_bytes
 * of the pool and is row_bytes long; the B rows of a block are contiguous.
 * num_sides is 2 for separate K and V objects, 1 for a single latent (MLA).
 * row_bytes is H_kv * head_dim * element size. layer_stride == 0 describes a
 * one-layer slot pool that every layer reuses (DualPath's per-layer HBM slot).
 * Requires num_sides >= 1, block_tokens >= 1, row_bytes >= 1, num_blocks >= 1,
 * strides >= 0 and block_stride >= block_tokens*row_bytes when num_blocks > 1. */
typedef struct {
    int32_t num_sides;
    int32_t block_tokens;
    int64_t row_bytes;
    int64_t block_stride;
    int64_t side_stride;
    int64_t layer_stride;
    int64_t num_blocks;
} kvm_pool_layout;

/* One sequence for kvm_pack_full / kvm_unpack_layer.
 *   block_table  device int32 array of at least ceil(num_tokens / block_tokens)
 *                entries; token t lives in block block_table[t / B], row t % B.
 *   full         device Full Block of this sequence, token-major
 *                [T][L][num_sides * row_bytes] (DualPath key-objects table: the
 *                [T, L, C_KV] view, C_KV = the K heads then the V heads). Token t,
 *                layer l, side s starts at t*token_stride + (l*S + s)*row_bytes.
 *   num_tokens   tokens to move: pack reads tokens [0, num_tokens) from the pool;
 *                unpack writes tokens [0, num_tokens) (the hit tokens) into their
 *                slots; every other slot byte is left as it was.
 *   token_stride bytes between consecutive tokens of `full`; 0 means dense
 *                (L * num_sides * row_bytes). Must be >= that dense size or 0. */
typedef struct {
    const int32_t* block_table;
    void* full;
    int64_t num_tokens;
    int64_t token_stride;
} kvm_seq;

/* One request for kvm_merge_layer (DualPath "two read paths": the hit slice and
 * the miss rows are concatenated by token). Rows are `row_bytes` long (C_KV
 * bytes); strides are in bytes between consecutive rows.
 *   hit   t_hit rows; hit + t*hit_stride. For the layer-l slice of a dense Full
 *         Block pass full + l*C_KV bytes and hit_stride = L*C_KV bytes.
 *   miss  t_miss rows; miss + i*miss_stride.
 *   out   t_hit + t_miss rows: out + t*out_stride receives hit row t for
 *         t < t_hit, and miss row t - t_hit after that. Row padding (bytes past
 *         row_bytes within out_stride) is left as it was.
 * A null pointer is allowed where its row count is 0. */
typedef struct {
    const void* hit;
    int64_t hit_stride;
    int64_t t_hit;
    const void* miss;
    int64_t miss_stride;
    int64_t t_miss;
    void* out;
    int64_t out_stride;
} kvm_merge_seq;

/* One contiguous object of kvm_batch_copy: nbytes from src_base + src_off to
 * dst_base + dst_off (Tutti reading notes, design 1, eq. 9: one entry per whole
 * object; offsets relative to a known base as in Mooncake's relocation).
 * 24 bytes; the array lives in DEVICE memory. */
typedef struct {
    uint64_t src_off;
    uint64_t dst_off;
    uint64_t nbytes;
} kvm_copy_desc;

/* KVM_ABI_VERSION of the built library. A caller compares it with the
 * KVM_ABI_VERSION it was compiled against before creating a context. */
int kvm_version(void);

/* Static text for a status code. Never NULL. */
const char* kvm_strerror(int status);

/* Create a context on HIP device `device` (the "initialize engine" step of
 * the transfer lifecycle in Mooncake Ascend Transports, USE_ASCEND_DIRECT:
 * initialize, register memory, transfer asynchronously, query completion,
 * finalize; here a transfer is a call below and its completion is the
 * caller's stream). It owns a device error counter, the batched copy's
 * scratch (sized for lists of 65,536 objects; it grows when a call needs
 * more) and 512 bytes of pinned host memory where the batched copy's kernels
 * leave each list shape's piece count (see kvm_batch_copy).
 * *out is set only on KVM_OK. Errors: KVM_EINVAL (out NULL, device < 0),
 * KVM_EHIP (no such device, runtime failure), KVM_ENOMEM. */
int kvm_create(int device, kvm_ctx** out);

/* The "finalize" step of the same lifecycle (Mooncake Ascend Transports,
 * USE_ASCEND_DIRECT): wait for the context's outstanding work, then free it.
 * NULL is a no-op. */
void kvm_destroy(kvm_ctx* ctx);

/* Pre-size the batched copy's scratch for up to max_descs copy objects per
 * call, so that later calls allocate nothing (the lifecycle's "register
 * memory" step, Mooncake Ascend Transports, USE_ASCEND_DIRECT: resources are
 * set up once, before the transfers that use them): 32 bytes per 64 objects
 * and 24 bytes per piece record, with room for max_descs pieces (objects of
 * up to 128 KiB). A call that needs more (more objects, or more pieces: a
 * call may need up to min(n_descs, dst_bytes / 16 KiB) + dst_bytes / 128 KiB
 * + 1) grows the scratch itself, to at least twice its size, without
 * waiting: the old buffer stays allocated until the next device
 * synchronisation below. This call synchronises the device when it resizes
 * the scratch or has such buffers to free, and frees them.
 * max_seqs, the sequences per call, needs no memory and is only range-checked
 * (at most 2^20). Errors: KVM_EINVAL (negative sizes), KVM_ERANGE, KVM_ENOMEM,
 * KVM_EHIP. */
int kvm_ctx_reserve(kvm_ctx* ctx, int64_t max_seqs, int64_t max_descs);

/* Pre-size the unpack tile-order scratch, as kvm_ctx_reserve does for the
 * batched copy (the same "register memory" step): every order slot of the context
 * (16) holds max_tiles entries, and the counting sort serves pools of up to
 * max_pool_blocks blocks. Later kvm_unpack_layer and kvm_unpack_merge_layer
 * calls whose launch batches (128 sequences each) hold at most max_tiles
 * block-table entries, on pools of at most max_pool_blocks blocks, allocate
 * no device memory (on one stream: the first call on a second stream takes
 * fresh order scratch, see kvm_unpack_layer). With kvm_ctx_reserve for the
 * batched copy this gives an allocation-free steady state. Synchronises the
 * device, frees replaced scratch and drops cached orders that it resizes. Uses 64 * max_tiles + 8 * max_pool_blocks bytes
 * (plus a small constant). Errors: KVM_EINVAL (null ctx, negative sizes),
 * KVM_ERANGE (max_tiles above 2^31 - 1, max_pool_blocks above 2^31),
 * KVM_ENOMEM, KVM_EHIP. */
int kvm_ctx_reserve_unpack(kvm_ctx* ctx, int64_t max_tiles, int64_t max_pool_blocks);

/* Device memory the context holds right now, in bytes: its error counter,
 * the batched-copy scratch, the unpack order scratch, and scratch set aside
 * until the next device synchronisation (see the waits convention above). It
 * changes only when a call grows, sets aside or frees that scratch. Errors: KVM_EINVAL
 * (null ctx or bytes). */
int kvm_ctx_device_bytes(const kvm_ctx* ctx, int64_t* bytes);

/* Workgroup budget: every later pack, unpack, merge, fused and batched-copy
 * launch through this context uses a grid of at most max_workgroups
 * workgroups, each of which loops over the tiles (or byte shares) that a
 * full-size grid would spread over more workgroups. The moves then occupy a
 * bounded share of the CUs, so that a layer's moves can run beside the
 * previous layer's compute on another stream (DualPath KV Loading, layerwise
 * Prefill; Tutti reading notes, design 2: I/O kernels kept to a few SMs
 * beside compute). The bytes written are the same for every budget.
 * 0 (the default) keeps the library's own grids: one workgroup per work item
 * for pack, unpack and the fused call, and for merge of rows under 2 KiB
 * (up to 4,194,303 workgroups, the most a dispatch of 1024-thread
 * workgroups can count; above that each takes several items); at most 16
 * workgroups per CU for merge of longer rows; for the batched copy one
 * 1024-thread workgroup per piece (at least 2 per CU). The destination-order sort that unpack
 * runs once per new set of block tables is not bounded (it touches 8 bytes
 * per tile). Applies to calls enqueued after it returns; calls already
 * enqueued keep their grids. Errors: KVM_EINVAL (null ctx, max_workgroups < 0). */
int kvm_ctx_set_max_workgroups(kvm_ctx* ctx, int32_t max_workgroups);

/* Debug mode: with enable != 0, every later unpack, fused and batched-copy
 * call first checks on the host the caller preconditions the kernels cannot
 * see, and returns KVM_ECHECK, with the offending entries named in
 * kvm_ctx_last_error, having enqueued nothing:
 *   kvm_unpack_layer, kvm_unpack_merge_layer: no valid block id appears
 *     twice among the block-table entries the call writes (all sequences);
 *   kvm_batch_copy: destination ranges are pairwise disjoint, and disjoint
 *     from every source range when the two buffers overlap.
 * Entries the kernels skip anyway (ids outside [0, num_blocks), objects
 * outside their buffer, zero-length objects) are not violations. A checked
 * call synchronises `stream` and copies the block tables or the descriptor
 * array to the host: it is for debugging, not the hot path. New contexts
 * start with checks on when the environment variable KVM_CHECK is "1".
 * Errors: KVM_EINVAL (null ctx). */
int kvm_ctx_set_checks(kvm_ctx* ctx, int32_t enable);

/* Text of the last HIP failure or check violation seen by this context ("" if
 * none). */
const char* kvm_ctx_last_error(const kvm_ctx* ctx);

/* Synchronise the context's device, then return in *count the number of
 * block-table entries (counted once per layer for pack) and copy objects that
 * device-side guards skipped since the previous call, and reset the counter.
 * Errors: KVM_EINVAL, KVM_EHIP. */
int kvm_take_device_errors(kvm_ctx* ctx, int64_t* count);

/* Pack (DualPath key-objects table, the persisted Full Block): for each
 * sequence, every token t < num_tokens, layer l < num_layers and side s:
 *     full[t][l][s] <- pool[l][s][block_table[t / B]][t % B]        (row_bytes)
 * One launch per 128 sequences; one workgroup per (sequence, block, layer)
 * tile.
 * n == 0, or sequences with num_tokens == 0, enqueue nothing for them.
 * Errors: KVM_EINVAL (null ctx/layout/pool/seqs with n > 0, a sequence with
 * null pointers and num_tokens > 0, bad layout or strides, n < 0,
 * num_layers < 1), KVM_ERANGE (n above 2^20, a tile above 2^31 bytes or
 * 2^31 work items in one launch), KVM_ENOMEM, KVM_EHIP. */
int kvm_pack_full(kvm_ctx* ctx, const kvm_pool_layout* layout, const void* pool,
                  int32_t num_layers, const kvm_seq* seqs, int32_t n, void* stream);

/* Unpack one layer (DualPath "two read paths": the layer-l slice of the Full
 * Block into the HBM layer slot): for each sequence, every token
 * t < num_tokens and side s:
 *     pool[layer][s][block_table[t / B]][t % B] <- full[t][layer][s]  (row_bytes)
 * Slot rows of tokens >= num_tokens (a partial last block shared with miss
 * tokens) are left as they were. One launch per 128 sequences; a work item
 * is one side of one or two consecutive blocks in ascending destination-block
 * order, one workgroup each. The
 * first call with a given set of sequence records sorts the blocks on the
 * stream (a counting sort over the pool's blocks, kept in the context for the
 * following layers; skipped when the pool has far more blocks than the call
 * has tiles). The context keeps 16 such orders; a new record set beyond that
 * replaces the least recently used one, after every launch that read it. While
 * all of a context's unpack and fused calls use one stream, stream order
 * provides that and nothing is recorded per call. The launches on that first
 * stream leave no events, so the first call on a second stream does not wait
 * for them: it sets every cached order and the sort's counters aside (they
 * stay allocated until the next device synchronisation, see the waits
 * convention above) and sorts into new ones, which it allocates. From then on
 * each call records an event that a later replacement waits for on the host.
 * Streams are told apart by handle: synchronize a stream before destroying it
 * if a context's launches on it may still be running.
 * Errors: as kvm_pack_full, plus KVM_ERANGE for layer outside
 * [0, num_layers) or more than 2048 sequences with tokens in one call, and
 * KVM_ECHECK (checks on, kvm_ctx_set_checks). */
int kvm_unpack_layer(kvm_ctx* ctx, const kvm_pool_layout* layout, void* pool,
                     int32_t num_layers, int32_t layer, const kvm_seq* seqs, int32_t n,
                     void* stream);

/* Merge one layer (DualPath "two read paths": concatenate hit and miss by
 * token into complete_layer[l] [T_all, C_KV]): for each request,
 *     out row t      <- hit row t             for t < t_hit
 *     out row t_hit+i <- miss row i           for i < t_miss
 * One launch per 128 requests. Errors: KVM_EINVAL (null ctx, row_bytes < 1,
 * negative counts or strides, a null pointer with a nonzero row count, n < 0),
 * KVM_ERANGE (n above 2^20, row_bytes of 2^31 or more), KVM_ENOMEM, KVM_EHIP. */
int kvm_merge_layer(kvm_ctx* ctx, int64_t row_bytes, const kvm_merge_seq* seqs, int32_t n,
                    void* stream);

/* One request for kvm_unpack_merge_layer: the union of its kvm_seq (the hit
 * tokens of the Full Block and the block table) and its kvm_merge_seq (the
 * miss rows and the complete_layer output). The hit rows are the layer slice
 * of `full`, so there is no separate hit pointer.
 *   block_table, full, t_hit, token_stride   as kvm_seq (num_tokens = t_hit)
 *   miss, miss_stride, t_miss                 as kvm_merge_seq
 *   out, out_stride                           as kvm_merge_seq (T_all rows) */
typedef struct {
    const int32_t* block_table;
    const void* full;
    int64_t t_hit;
    int64_t token_stride;
    const void* miss;
    int64_t miss_stride;
    int64_t t_miss;
    void* out;
    int64_t out_stride;
} kvm_layer_seq;

/* Unpack and merge one layer in one pass over the hit slice (DualPath "two
 * read paths": the layer's hit slice goes both into the HBM layer slot and,
 * concatenated with the miss rows, into complete_layer[l]). Exactly the result
 * of kvm_unpack_layer(layer) on {block_table, full, t_hit, token_stride}
 * followed by kvm_merge_layer(row_bytes = num_sides*row_bytes) on
 * {hit = full + layer*num_sides*row_bytes, hit_stride = token_stride (dense if
 * 0), t_hit, miss, miss_stride, t_miss, out, out_stride}, but each hit row is
 * read once: 3*H + 2*M bytes move instead of 4*H + 2*M. Launches: one fused
 * kernel per 128 requests with hit rows: their tiles (in destination-block
 * order, as kvm_unpack_layer), then their miss rows as its last work items.
 * Miss rows of requests with no hit rows, or whose miss address or stride
 * would force narrower moves on the hit rows, take one merge launch of their
 * own.
 * Errors: the union of kvm_unpack_layer's and kvm_merge_layer's (KVM_ECHECK
 * included). */
int kvm_unpack_merge_layer(kvm_ctx* ctx, const kvm_pool_layout* layout, void* pool,
                           int32_t num_layers, int32_t layer, const kvm_layer_seq* seqs,
                           int32_t n, void* stream);

/* Batched copy of many non-contiguous objects in one launch sequence
 * (Tutti "pseudo-code 1": one submission per layer for thousands of objects;
 * Mooncake Ascend Transports, USE_ASCEND: batching non-contiguous 128 KB blocks):
 * for every k < n_descs,
 *     dst_base[dst_off_k .. dst_off_k + nbytes_k) <- src_base[src_off_k .. + nbytes_k)
 * descs is a DEVICE array of n_descs kvm_copy_desc. dst_bytes and src_bytes are
 * the sizes of the two buffers; an object outside its buffer is skipped and
 * counted (kvm_take_device_errors). Zero-length objects are no-ops. dst_base and
 * src_base may be the same buffer.
 * How: objects of at least 16 KiB whose source, destination and length are
 * multiples of 16 bytes are cut into pieces of at most 128 KiB, one 1024-thread
 * workgroup each; all other objects are shared evenly by the device's
 * wavefronts. A list of more than 64 objects first runs a metadata pass (one
 * launch up to 65,536 objects, three above) that sums, scans and records the
 * pieces in the context's scratch; a list of at most 64 objects is copied by
 * one launch that uses no scratch (it allocates nothing and orders itself
 * after no other stream's copy). The number of pieces is known only on the
 * device: the metadata pass leaves it in pinned host memory under the call's
 * list shape (n_descs and the two buffers, address and size), and the next
 * call of that shape sizes its grid from it without waiting for the device;
 * the first call of a shape guesses (one piece per object; for a list of one
 * object, as many pieces as the smaller buffer holds), and then loops over
 * the pieces its grid does not hold (same result, slower). When the previous
 * call of the shape found every object one piece, the call runs one
 * workgroup per object with no metadata pass (no scratch); an object that is
 * not one piece then still moves, and the shape goes back to the metadata
 * pass at its next call.
 * Objects are taken in list order: a list sorted by destination offset copies
 * 1-4 % faster on MI355X (concurrent workgroups then write neighbouring
 * objects), so a caller that builds its list on the host may sort it.
 * The first call with scratch on a second stream does not wait for the first
 * stream's copies (they left no events): it sets the scratch aside (allocated
 * until the next device synchronisation, see the waits convention above) and
 * takes a new one. From then on each call with scratch records an event, and
 * a call on another stream than the previous one waits, on the device, for
 * that call.
 * Errors: KVM_EINVAL (null ctx, null descs/bases with n_descs > 0, n_descs < 0),
 * KVM_ERANGE (n_descs above 2^32), KVM_ENOMEM, KVM_EHIP, KVM_ECHECK (checks on). */
int kvm_batch_copy(kvm_ctx* ctx, void* dst_base, uint64_t dst_bytes, const void* src_base,
                   uint64_t src_bytes, const kvm_copy_desc* descs, int64_t n_descs,
                   void* stream);

/* The largest n_descs kvm_batch_copy_noalloc accepts (2^25 - 64 objects: 2^19 - 1 groups of 64). */
#define KVM_NOALLOC_MAX_DESCS ((INT64_C(1) << 25) - 64)

/* For callers that cannot allocate device memory during a call (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * kvm_batch_copy with its scratch in a static device array of 16 MiB per GPU
 * (the list's sums and bases, 32 bytes per 64 objects, then its piece records,
 * 24 bytes each), which the library reserves for the life of the process on
 * every device it runs on. A list whose piece records might not fit (more
 * than the array holds after the sums, by the bound given for
 * kvm_ctx_reserve) sends every object to the wavefront shares instead.
 * Same arguments, result and error behaviour as kvm_batch_copy, except:
 *   - it calls no hipMalloc, hipFree or other allocating routine, records no
 *     event and never waits on another stream;
 *   - lists longer than KVM_NOALLOC_MAX_DESCS objects return KVM_ERANGE;
 *   - every call on one GPU, from any context or stream, shares that GPU's
 *     array, which keeps the last call's contents: calls that overlap on one
 *     GPU (on two streams, or from two threads) race and give an unspecified
 *     result. Order them on one stream, or synchronise between them;
 *   - the debug checks of kvm_ctx_set_checks are not applied.
 * The array's address is taken when the context is created (kvm_create).
 * The call may be captured into a HIP graph: its launch configuration (the
 * grid, or one workgroup per object) is fixed when it is captured, and every
 * configuration copies any list of the captured length correctly, so a replay
 * copies the descriptors as they are at that replay. Replays share the
 * static array like any other call. */
int kvm_batch_copy_noalloc(kvm_ctx* ctx, void* dst_base, uint64_t dst_bytes,
                           const void* src_base, uint64_t src_bytes,
                           const kvm_copy_desc* descs, int64_t n_descs, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVM_H */
