// kernels.hip -- gfx950 (CDNA4) kernels of libkvmove.
//
// Every kernel here is a byte mover: no value is read as a number. They are
// bound by HBM bandwidth, so the design is about keeping enough 16-byte loads
// in flight per CU, keeping every lane busy on ragged rows, and never writing
// a partial cache line that a full row would cover:
//
//   k_pack / k_unpack /  one workgroup per work item. A pack item is
//   k_unpack_merge      (sequence, block, layer); an unpack or fused item is
//                       one side of two consecutive tiles in destination
//                       order (of one tile when a tile exceeds 2048 16-byte
//                       units).
//                       With a workgroup budget below the item count, the
//                       grid is the budget and workgroup i takes items i,
//                       i + grid, i + 2*grid, ... (this bounds how many CUs
//                       the moves occupy while other work shares the GPU).
//                       An item's rows are flattened into one index space of
//                       `unit`-byte elements so that a 1152-byte MLA row or a
//                       256-byte tiny row keeps every lane busy; element ->
//                       (row, side, column) for pack, (row, column) for the
//                       others, uses multiply-high division by invariant
//                       integers.
//   k_merge             a tile is (request, chunk of rows); a row comes from
//                       the strided hit slice or from the miss rows. For rows
//                       of 2 KiB and more the grid is capped (16 workgroups
//                       per CU) and each workgroup walks tiles i, i + grid,
//                       ...; shorter rows take one workgroup per tile.
//   k_bc_*              batched copy: per-group byte sums (64 objects per
//                       wavefront), one exclusive scan (one workgroup does
//                       both for lists of up to 1,024 groups), then a fixed
//                       grid in which every wavefront copies an equal share
//                       of the total bytes, walking the objects its share
//                       covers.
//
// Page notation (DualPath KV Loading, key-objects table; Tutti reading notes,
// prerequisites 3 and 5): T tokens, L layers, C_KV = sides * row_bytes per
// token-layer row, B tokens per block, block table bt.
#include "kvm_internal.h"

#include <algorithm>
#include <mutex>

namespace kvm {

// 16-byte vectors each lane of a batched-copy wavefront keeps in flight.
constexpr int kCopyUnroll = 8;

FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
    f.s = l;
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f)
{
    const uint32_t hi = __umulhi(n, f.m);
    return uint32_t((uint64_t(hi) + n) >> f.s);
}

template <int U> struct Unit;
template <> struct Unit<16> { typedef uint32_t T __attribute__((ext_vector_type(4))); };
template <> struct Unit<8> { typedef uint32_t T __attribute__((ext_vector_type(2))); };
template <> struct Unit<4> { typedef uint32_t T; };
template <> struct Unit<2> { typedef uint16_t T; };
template <> struct Unit<1> { typedef uint8_t T; };

typedef Unit<16>::T V16;

// Streaming cache policy. Every payload byte is read once and written once,
// so loads are non-temporal, and 16-byte stores carry "sc1 nt" (on gfx950,
// sc1 without sc0 is agent (device) scope; system scope would be "sc0 sc1";
// nt marks the line as streaming): measured on MI355X, this mix moves 3-4 %
// more copy traffic through HBM than default-policy stores, and more for
// scattered objects. Stores into pinned host memory (a host-resident Full
// Block or complete_layer) become visible to the host through the release at
// the end of the kernel, not through the store's own scope. Narrower units
// (unaligned edge cases) use default stores.
template <class V>
__device__ __forceinline__ V ld(const V* p)
{
    return __builtin_nontemporal_load(p);
}

template <class V>
__device__ __forceinline__ void st(V* p, V v)
{
    *p = v;
}

template <>
__device__ __forceinline__ void st<V16>(V16* p, V16 v)
{
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt" ::"v"(p), "v"(v) : "memory");
}

// Index of the record whose tile range holds `tile`: the last i with
// tile0[i] <= tile. The search index is the same in every lane, so each probe
// is one scalar load from the kernel-argument segment.
__device__ __forceinline__ int32_t find_record(const int64_t* tile0, int32_t n, int64_t tile)
{
    int32_t lo = 0, hi = n - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (tile0[mid] <= tile) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ bool bad_block(int32_t blk, int64_t num_blocks)
{
    return blk < 0 || int64_t(blk) >= num_blocks;
}

// A work item of a batch whose records carry block tables: its record si,
// the block-table entry b it covers, the block id found there, the layer l
// (pack only) and the side (unpack and the fused kernel take one side of a
// block per work item). per = tiles per block-table entry (L for pack, else 1).
struct TileAt {
    int32_t si;
    int32_t l;
    int32_t side;
    int64_t b;
    int32_t blk;
};

template <class Batch>
__device__ __forceinline__ TileAt tile_at(const Batch& batch, int32_t per, int64_t tile,
                                          int32_t side)
{
    TileAt t;
    t.si = find_record(batch.tile0, batch.n, tile);
    const int64_t rem = tile - batch.tile0[t.si];
    t.b = per == 1 ? rem : rem / per;
    t.l = int32_t(rem - t.b * per);
    t.side = side;
    t.blk = batch.rec[t.si].block_table[t.b];
    return t;
}

// The tiles a work item covers: G consecutive entries of the tile order (the
// last item of a launch may hold fewer), all on the same side.
template <int G>
struct Item {
    TileAt t[G];
    int32_t count;
};

template <int G>
struct TileIdx {
    int64_t v[G];  // tile indices; -1 past the launch's last tile
};

// Work item i is side i % sides of tiles order[G*p .. G*p + G) with
// p = i / sides (a null order means tiles G*p ..); workgroup blockIdx.x takes
// items blockIdx.x, + grid, ... Under a workgroup budget one workgroup copies
// many items in turn, so the next item's records and block ids are fetched
// before the current item is copied, and the order entries one item further
// ahead: the dependent metadata loads then overlap a copy instead of sitting
// between two. With one workgroup per item the loop body runs once.
template <int G, class Batch, class Body>
__device__ __forceinline__ void walk_items(const Batch& batch, int32_t per, int32_t sides,
                                           const int32_t* __restrict__ order, Body body)
{
    const int64_t nt = batch.tile0[batch.n];
    const int64_t n = (G == 1 ? nt : (nt + G - 1) / G) * sides;
    const int64_t grid = gridDim.x;
    auto side_of = [&](int64_t i) {
        return sides == 1 ? 0 : sides == 2 ? int32_t(i & 1) : int32_t(i % sides);
    };
    auto tiles_of = [&](int64_t i) {
        const int64_t p = (sides == 1 ? i : sides == 2 ? (i >> 1) : i / sides) * G;
        TileIdx<G> x;
#pragma unroll
        for (int q = 0; q < G; ++q)
            x.v[q] = p + q < nt ? (order ? int64_t(order[p + q]) : p + q) : -1;
        return x;
    };
    auto item_at = [&](const TileIdx<G>& x, int32_t side) {
        Item<G> it;
        it.count = 0;
#pragma unroll
        for (int q = 0; q < G; ++q)
            if (x.v[q] >= 0) {
                it.t[q] = tile_at(batch, per, x.v[q], side);
                it.count = q + 1;
            }
        return it;
    };
    int64_t i = blockIdx.x;
    if (i >= n) return;
    Item<G> cur = item_at(tiles_of(i), side_of(i));
    TileIdx<G> next = tiles_of(i + grid < n ? i + grid : i);
    for (;;) {
        const bool more = i + grid < n;
        Item<G> nxt = cur;
        if (more) nxt = item_at(next, side_of(i + grid));
        const int64_t j = i + 2 * grid;
        const TileIdx<G> after = tiles_of(j < n ? j : i);
        body(cur);
        if (!more) break;
        cur = nxt;
        next = after;
        i += grid;
    }
}

// One tile per work item.
template <class Batch, class Body>
__device__ __forceinline__ void walk_tiles(const Batch& batch, int32_t per, int32_t sides,
                                           const int32_t* __restrict__ order, Body body)
{
    walk_items<1>(batch, per, sides, order, [&](const Item<1>& it) { body(it.t[0]); });
}

// Copy the `total` unit-sized elements of one work item with a workgroup of BS
// threads: every thread issues UNR loads, then UNR stores, so a workgroup keeps
// BS*UNR*U bytes in flight. addr(j, src, dst) names element j's two addresses;
// consecutive j within a row are consecutive bytes of it, so a wavefront's 64
// lanes touch adjacent units except where a row ends. total is at most
// INT32_MAX (the host checks tile sizes), so no index below wraps. Which
// elements a wavefront takes per batch:
//   WAVE_MAJOR = false: element k of thread t is base + k*BS + t (a wavefront's
//                       UNR pieces are BS elements apart);
//   WAVE_MAJOR = true:  each wavefront owns 64*UNR consecutive elements.
template <int U, int BS, int UNR, bool WAVE_MAJOR, class Addr>
__device__ __forceinline__ void copy_elements(uint32_t total, Addr addr)
{
    typedef typename Unit<U>::T V;
    constexpr uint32_t kStep = WAVE_MAJOR ? 64 : BS;
    const uint32_t first =
        WAVE_MAJOR ? (threadIdx.x >> 6) * (64 * UNR) + (threadIdx.x & 63) : threadIdx.x;
    // in wave-major order a wavefront's first element may exceed a thread's
    // row of the batch, so iterate over whole batches
    const uint32_t limit = WAVE_MAJOR ? total + BS * UNR : total;
    for (uint32_t base = first; base < limit; base += BS * UNR) {
        V v[UNR];
        char* dp[UNR];
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const uint32_t j = base + k * kStep;
            if (j < total) {
                const char* sp;
                addr(j, sp, dp[k]);
                v[k] = ld(reinterpret_cast<const V*>(sp));
            }
        }
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const uint32_t j = base + k * kStep;
            if (j < total) st(reinterpret_cast<V*>(dp[k]), v[k]);
        }
    }
}

// Workgroup shapes and element orders, chosen by measurement on MI355X (all
// variants timed in one process on the same buffers, interleaved): pack and
// merge keep a whole tile in flight per workgroup (64 KiB; about 50 KiB for
// merge rows under 2 KiB, with 1024 x 8 slots: 1024 x 4 would need two
// passes and loses 6 %), pack in wave-major order (+2.4 % over
// thread-major), merge in thread-major order (wave-major costs it 18 %).
// Unpack and the fused kernel, whose stores land on scattered pool objects,
// take two tiles per work item and, for tiles above 2048 units (a 72 KiB MLA
// block), one tile per item at 1024 x 8 (unpack: 6.11 TB/s against 5.53 at
// 576 x 8; fused: +7 %; 768 x 6 and 512 x 9, an exact fit, lose 7 %), the
// fused kernel then with split stores. Pairs of more than 3072 units (Llama's
// 32 KiB block sides) take 1024 x 4, one pass: 768 x 4 costs unpack 4.5-11 %
// (two boxes, in one process and over alternating processes) and the fused
// layer 0.4-1.1 %; 1024 x 4 pairs beat one tile per item at 576 x 8 by
// 1.2-1.6 %. Pairs of 1025-3072 units (16-18 KiB block sides: 64-wide heads,
// MLA rows, 8-token blocks) take 768 x 4, 33-47 % ahead of 1024 x 4 for
// unpack and up to 17 % for the fused kernel; 576, 640 and 896 threads lose
// 5-35 %. No occupancy cap helps either.
constexpr int kPackBS = 1024, kPackUnroll = 4;
constexpr bool kPackWaveMajor = true;
// Smaller pack tiles take smaller workgroups, so that most slots of a pass
// hold an element: 768 threads for tiles of 1537-3072 units (a 32 KiB tile:
// +5 % over 1024 x 4 on 64-wide heads and on Llama with 8-token blocks), 512
// for 1536 units or fewer (MLA's 18 KiB tile with 16-token blocks: +62 %).
// Llama's 64 KiB tiles keep 1024 x 4 (every smaller shape loses 5-10 %).
// Tiles of at most 768 units take 256 threads (8 KiB tiles of 512-byte rows
// with 16-token blocks: +40 %); at 1024 units 256 x 4 was +6 % on one shape
// and -2 % on another, so those keep 512.
constexpr int kPackMidBS = 768, kPackSmallBS = 512, kPackTinyBS = 256;
constexpr int64_t kPackMidUnits = 3072, kPackSmallUnits = 1536, kPackTinyUnits = 768;
constexpr int kMergeBS = 1024, kMergeUnroll = 4;
constexpr bool kMergeWaveMajor = false;
constexpr int kMergeWideUnroll = 8;  // short rows: ~50 KiB tiles, 1024 x 8 slots
constexpr int kUnpackBS = 768, kUnpackUnroll = 4;
constexpr int kUnpackPairBS = 1024;  // pairs above 768 x 4 units, as kFusedPairBS
constexpr bool kUnpackWaveMajor = false;
constexpr int kUnpackWideBS = 1024, kUnpackWideUnroll = 8;
constexpr int64_t kUnpackWideItem = 2048;  // 16-byte units per tile above which unpack
                                           // and the fused kernel take the wide shape
constexpr int kFusedBS = 768, kFusedUnroll = 4;
constexpr int kFusedPairBS = 1024;  // pairs above 768 x 4 units (16-byte units)
// A pair of 8 KiB tiles (at most 1024 units) leaves most of a 768 x 4 pass
// idle: unpack takes 256 x 4 for it (+45-52 % on 512-byte rows with 16-token
// blocks and 1 KiB rows with 8-token blocks), the fused kernel 512 x 4 (+2 to
// +19 %; 256 x 4 ranged from -1 to +21 %). On 16 KiB tiles 512 x 4 loses 3-4 %
// to 768 x 4, so the rule stops at 1024 units.
constexpr int kUnpackSmallBS = 256, kFusedSmallBS = 512;
constexpr int64_t kSmallPairUnits = 1024;
constexpr int kFusedWideBS = 1024, kFusedWideUnroll = 8;

// ---------------------------------------------------------------- pack ---
// full[t][l][s] <- pool[l][s][bt[t / B]][t % B] for the tokens of one block
// and one layer. Element j of the tile: row r = j / (S*V), q = j % (S*V) is the
// unit offset inside the token's C_KV row, side = q / V, column c = q % V.
template <int U, int BS, int UNR, bool WM>
__global__ __launch_bounds__(BS) void k_pack(PoolGeom g, const char* __restrict__ pool,
                                             int32_t num_layers, const SeqBatch batch,
                                             FastDiv div_q, FastDiv div_v,
                                             unsigned long long* err)
{
    walk_tiles(batch, num_layers, 1, nullptr, [&](const TileAt& t) {
        const SeqRec& s = batch.rec[t.si];
        const int64_t b = t.b;
        const int32_t l = t.l;
        const int32_t blk = t.blk;
        if (bad_block(blk, g.num_blocks)) {
            if (threadIdx.x == 0) atomicAdd(err, 1ull);
            return;
        }
        const int64_t t0 = b * g.block_tokens;
        const uint32_t rows = uint32_t(min(int64_t(g.block_tokens), s.num_tokens - t0));
        const char* src = pool + l * g.layer_stride + blk * g.block_stride;
        char* dst = const_cast<char*>(s.full) + t0 * s.token_stride +
                    int64_t(l) * g.sides * g.row_bytes;
        copy_elements<U, BS, UNR, WM>(rows * div_q.d, [&](uint32_t j, const char*& sp, char*& dp) {
            const uint32_t r = fdiv(j, div_q);
            const uint32_t q = j - r * div_q.d;
            const uint32_t side = fdiv(q, div_v);
            const uint32_t c = q - side * div_v.d;
            sp = src + side * g.side_stride + int64_t(r) * g.row_bytes + int64_t(c) * U;
            dp = dst + int64_t(r) * s.token_stride + int64_t(q) * U;
        });
    });
}

// -------------------------------------------------------------- unpack ---
// pool[layer][side][bt[t / B]][t % B] <- full[t][layer][side] for the tokens
// of a block below num_tokens. A work item is one side of G consecutive tiles
// of the order: B strided row pieces read and one contiguous object written
// per tile. Tiles are taken in order[] (sorted by destination block id,
// k_order_*), so the object stores of concurrently running workgroups ascend
// through the pool instead of landing at random, and the G objects of one
// item are often adjacent. A null order keeps the tiles' own order. Element j
// of an item belongs to its first tile below the first tile's element count,
// else to the second; within a tile it is row j / V, unit column j % V.
//
// Measured on MI355X (Llama block sides of 32 KiB): one side per item is
// 7.6 % faster than both sides of a block (each workgroup then writes one
// object, not two far apart), and two consecutive tiles per item another
// 1.2-1.6 % faster than one (then at 1024 x 4; 512 x 8, 1024 x 2 and three
// or four tiles per item are slower), and 768 threads faster again.

// The G tiles' source and destination bases and element counts, and the
// error count for tiles with bad block ids (once per tile, on side 0).
template <int G>
struct ItemSpan {
    const char* src[G];
    char* dst[G];
    char* out[G];
    int64_t src_stride[G];
    int64_t out_stride[G];
    uint32_t first_end;  // elements of the first tile
    uint32_t total;
};

template <int G, class Batch>
__device__ __forceinline__ ItemSpan<G> item_span(const PoolGeom& g, char* pool, int32_t layer,
                                                 const Batch& batch, const Item<G>& it,
                                                 uint32_t units, unsigned long long* err)
{
    static_assert(G == 1 || G == 2, "one or two tiles per work item");
    ItemSpan<G> sp;
    uint32_t count[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
        count[q] = 0;
        sp.src[q] = nullptr;
        sp.dst[q] = nullptr;
        sp.out[q] = nullptr;
        sp.src_stride[q] = 0;
        sp.out_stride[q] = 0;
        if (q >= it.count) continue;
        const TileAt& t = it.t[q];
        if (bad_block(t.blk, g.num_blocks)) {
            if (threadIdx.x == 0 && t.side == 0) atomicAdd(err, 1ull);
            continue;
        }
        const auto& s = batch.rec[t.si];
        const int64_t t0 = t.b * g.block_tokens;
        count[q] = uint32_t(min(int64_t(g.block_tokens), s.num_tokens - t0)) * units;
        sp.src[q] = s.full + t0 * s.token_stride + (int64_t(layer) * g.sides + t.side) * g.row_bytes;
        sp.dst[q] = pool + layer * g.layer_stride + t.side * g.side_stride + t.blk * g.block_stride;
        sp.src_stride[q] = s.token_stride;
        if constexpr (Batch::kHasOut) {
            sp.out[q] = s.out + t0 * s.out_stride + int64_t(t.side) * g.row_bytes;
            sp.out_stride[q] = s.out_stride;
        }
    }
    sp.first_end = count[0];
    sp.total = G == 1 ? count[0] : count[0] + count[G - 1];
    return sp;
}

template <int U, int BS, int UNR, bool WM, int G>
__global__ __launch_bounds__(BS) void k_unpack(PoolGeom g, char* __restrict__ pool, int32_t layer,
                                               const SeqBatch batch, const int32_t* __restrict__ order,
                                               FastDiv div_v, unsigned long long* err)
{
    walk_items<G>(batch, 1, g.sides, order, [&](const Item<G>& it) {
        const ItemSpan<G> sp = item_span<G>(g, pool, layer, batch, it, div_v.d, err);
        copy_elements<U, BS, UNR, WM>(sp.total, [&](uint32_t j, const char*& s, char*& d) {
            const bool second = G == 2 && j >= sp.first_end;
            const uint32_t jj = second ? j - sp.first_end : j;
            const uint32_t r = fdiv(jj, div_v);
            const uint32_t c = jj - r * div_v.d;
            s = (second ? sp.src[G - 1] : sp.src[0]) +
                int64_t(r) * (second ? sp.src_stride[G - 1] : sp.src_stride[0]) + int64_t(c) * U;
            d = (second ? sp.dst[G - 1] : sp.dst[0]) + int64_t(r) * g.row_bytes + int64_t(c) * U;
        });
    });
}

// ---------------------------------------------------- unpack + merge ---
// The hit rows of one layer, read once and stored twice: into the block-table
// slots (as k_unpack) and into the request's output rows t0..t0+rows (as the
// hit part of k_merge). Same work items, order and element order as k_unpack;
// the second store of element j (row r, column c) of side s goes to
// out + (t0 + r)*out_stride + s*row_bytes + c*U. SPLIT issues a batch's pool
// stores before its output stores rather than the two stores of each element
// in turn (measured on MI355X: +2-4.5 % on 1152- and 1024-byte MLA rows,
// -1.2 % on Llama's 2 KiB block sides). Two tiles per item: +1.2 % on Llama.
template <int U, int BS, int UNR, bool SPLIT, int G>
__global__ __launch_bounds__(BS) void k_unpack_merge(PoolGeom g, char* __restrict__ pool,
                                                     int32_t layer, const LayerBatch batch,
                                                     const int32_t* __restrict__ order,
                                                     FastDiv div_v, unsigned long long* err)
{
    typedef typename Unit<U>::T V;
    walk_items<G>(batch, 1, g.sides, order, [&](const Item<G>& it) {
        const ItemSpan<G> sp = item_span<G>(g, pool, layer, batch, it, div_v.d, err);
        const uint32_t total = sp.total;
        for (uint32_t base = threadIdx.x; base < total; base += BS * UNR) {
            V v[UNR];
            char* dp[UNR];
            char* op[UNR];
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const uint32_t j = base + k * BS;
                if (j < total) {
                    const bool second = G == 2 && j >= sp.first_end;
                    const uint32_t jj = second ? j - sp.first_end : j;
                    const uint32_t r = fdiv(jj, div_v);
                    const uint32_t c = jj - r * div_v.d;
                    const int q = second ? G - 1 : 0;
                    v[k] = ld(reinterpret_cast<const V*>(sp.src[q] + int64_t(r) * sp.src_stride[q] +
                                                         int64_t(c) * U));
                    dp[k] = sp.dst[q] + int64_t(r) * g.row_bytes + int64_t(c) * U;
                    op[k] = sp.out[q] + int64_t(r) * sp.out_stride[q] + int64_t(c) * U;
                }
            }
            if constexpr (SPLIT) {
#pragma unroll
                for (int k = 0; k < UNR; ++k)
                    if (base + k * BS < total) st(reinterpret_cast<V*>(dp[k]), v[k]);
#pragma unroll
                for (int k = 0; k < UNR; ++k)
                    if (base + k * BS < total) st(reinterpret_cast<V*>(op[k]), v[k]);
            } else {
#pragma unroll
                for (int k = 0; k < UNR; ++k) {
                    const uint32_t j = base + k * BS;
                    if (j < total) {
                        st(reinterpret_cast<V*>(dp[k]), v[k]);
                        st(reinterpret_cast<V*>(op[k]), v[k]);
                    }
                }
            }
        }
    });
}

// --------------------------------------------------------------- merge ---
// out row t <- hit row t (t < t_hit) or miss row t - t_hit, for one chunk of
// rows_per_tile rows of one request. Element j: row r = j / V, column j % V.
template <int U, int BS, int UNR, bool WM>
__global__ __launch_bounds__(BS) void k_merge(int32_t rows_per_tile, const MergeBatch batch,
                                              FastDiv div_v)
{
    const int64_t ntiles = batch.tile0[batch.n];
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int32_t si = find_record(batch.tile0, batch.n, tile);
        const MergeRec m = batch.rec[si];
        const int64_t row0 = (tile - batch.tile0[si]) * rows_per_tile;
        const int64_t t_all = m.t_hit + m.t_miss;
        const uint32_t rows = uint32_t(min(int64_t(rows_per_tile), t_all - row0));
        copy_elements<U, BS, UNR, WM>(rows * div_v.d, [&](uint32_t j, const char*& sp, char*& dp) {
            const uint32_t r = fdiv(j, div_v);
            const uint32_t c = j - r * div_v.d;
            const int64_t row = row0 + r;
            sp = (row < m.t_hit ? m.hit + row * m.hit_stride
                                : m.miss + (row - m.t_hit) * m.miss_stride) + int64_t(c) * U;
            dp = m.out + row * m.out_stride + int64_t(c) * U;
        });
    }
}

// -------------------------------------------------- unpack tile order ---
// A counting sort of one launch batch's unpack tiles by destination block id.
// Measured on MI355X: writing the scattered 32 KiB pool objects in ascending
// block order, while the Full Block rows are read in whatever order that
// gives, is 21 % faster than the tables' own order (one item per block side).
// Tiles with equal keys may come out in any order; only repeated or bad ids
// share a key. The sort is robust to any table contents:
// an id outside [0, N) gets key N (its tile is skipped by k_unpack anyway),
// and repeated ids share a key, so the result is always a permutation of the
// batch's tiles.

__device__ __forceinline__ int64_t order_key(const SeqRec& s, int64_t b, int64_t num_blocks)
{
    const int32_t blk = s.block_table[b];
    return bad_block(blk, num_blocks) ? num_blocks : int64_t(blk);
}

__global__ __launch_bounds__(256) void k_order_zero(uint32_t* __restrict__ cnt, int64_t n)
{
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
        cnt[i] = 0;
}

// grid: x = chunks of 256 tiles of one record, y = record
__global__ __launch_bounds__(256) void k_order_count(const SeqBatch batch, int64_t num_blocks,
                                                     uint32_t* __restrict__ cnt)
{
    const int32_t si = blockIdx.y;
    const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (b >= batch.tile0[si + 1] - batch.tile0[si]) return;
    atomicAdd(&cnt[order_key(batch.rec[si], b, num_blocks)], 1u);
}

__global__ __launch_bounds__(256) void k_order_place(const SeqBatch batch, int64_t num_blocks,
                                                     uint32_t* __restrict__ cursor,
                                                     int32_t* __restrict__ order)
{
    const int32_t si = blockIdx.y;
    const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (b >= batch.tile0[si + 1] - batch.tile0[si]) return;
    const uint32_t pos = atomicAdd(&cursor[order_key(batch.rec[si], b, num_blocks)], 1u);
    order[pos] = int32_t(batch.tile0[si] + b);
}

// One workgroup: out[i] = sum of in[0..i) for i < n, and out[n] = the total.
template <class T>
__global__ __launch_bounds__(1024) void k_exclusive_scan(const T* __restrict__ in,
                                                         T* __restrict__ out, int64_t n)
{
    __shared__ T wave_total[16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t per = (n + 1023) / 1024;
    const int64_t a = min(n, int64_t(tid) * per);
    const int64_t b = min(n, a + per);
    T local = 0;
    for (int64_t i = a; i < b; ++i) local += in[i];
    T x = local;  // inclusive scan across the wavefront
    for (int o = 1; o < 64; o <<= 1) {
        const T y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wave_total[wid] = x;
    __syncthreads();
    T before = 0;
    for (int w = 0; w < wid; ++w) before += wave_total[w];
    T run = before + x - local;
    for (int64_t i = a; i < b; ++i) {
        out[i] = run;
        run += in[i];
    }
    if (tid == 1023) out[n] = before + x;
}

// ---------------------------------------------------------- batch copy ---

// Bytes object k contributes: its length, or 0 when it does not lie inside
// both buffers (then it is skipped everywhere).
__device__ __forceinline__ uint64_t object_bytes(const CopyDesc& x, uint64_t src_bytes,
                                                 uint64_t dst_bytes)
{
    const bool ok = x.src_off <= src_bytes && x.nbytes <= src_bytes - x.src_off &&
                    x.dst_off <= dst_bytes && x.nbytes <= dst_bytes - x.dst_off;
    return ok ? x.nbytes : 0;
}

// One wavefront per group of 64 objects: the group's byte count.
__global__ __launch_bounds__(kBlock) void k_bc_group_sums(const CopyDesc* __restrict__ descs,
                                                          int64_t n, uint64_t src_bytes,
                                                          uint64_t dst_bytes,
                                                          uint64_t* __restrict__ group_sum,
                                                          int64_t ngroups,
                                                          unsigned long long* err)
{
    const int lane = threadIdx.x & 63;
    const int64_t grp = int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (grp >= ngroups) return;
    const int64_t k = grp * kDescGroup + lane;
    unsigned long long len = 0;
    if (k < n) {
        const CopyDesc x = descs[k];
        len = object_bytes(x, src_bytes, dst_bytes);
        if (len != x.nbytes) atomicAdd(err, 1ull);
    }
    for (int o = 32; o > 0; o >>= 1) len += __shfl_xor(len, o);
    if (lane == 0) group_sum[grp] = len;
}

// Lists of at most kSmallGroups groups take one workgroup for both steps:
// its 16 wavefronts sum groups w, w + 16, ... (one coalesced load of 64
// descriptors per group, four groups in flight per wavefront), then it scans
// the sums, writing what k_bc_group_sums and k_exclusive_scan write together:
// group_base[g] = the bytes of groups before g, group_base[ngroups] = total.
// Per-layer restore calls and small calls then start their copy one launch
// sooner.
constexpr int64_t kSmallGroups = 1024;
__global__ __launch_bounds__(1024) void k_bc_sums_scan(const CopyDesc* __restrict__ descs,
                                                       int64_t n, uint64_t src_bytes,
                                                       uint64_t dst_bytes,
                                                       uint64_t* __restrict__ group_base,
                                                       int64_t ngroups, unsigned long long* err)
{
    __shared__ unsigned long long sums[kSmallGroups];
    __shared__ unsigned long long wave_total[16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    for (int64_t g0 = wid; g0 < ngroups; g0 += 64) {
        CopyDesc x[4];
        unsigned long long len[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t k = (g0 + 16 * q) * kDescGroup + lane;
            x[q] = CopyDesc{0, 0, 0};
            if (g0 + 16 * q < ngroups && k < n) x[q] = descs[k];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            len[q] = object_bytes(x[q], src_bytes, dst_bytes);
            if (len[q] != x[q].nbytes) atomicAdd(err, 1ull);
            for (int o = 32; o > 0; o >>= 1) len[q] += __shfl_xor(len[q], o);
            if (lane == 0 && g0 + 16 * q < ngroups) sums[g0 + 16 * q] = len[q];
        }
    }
    __syncthreads();
    const unsigned long long v = tid < ngroups ? sums[tid] : 0;
    unsigned long long x = v;  // inclusive scan across the wavefront
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wave_total[wid] = x;
    __syncthreads();
    unsigned long long before = 0;
    for (int w = 0; w < wid; ++w) before += wave_total[w];
    if (tid < ngroups) group_base[tid] = before + x - v;
    if (tid == 1023) group_base[ngroups] = before + x;
}

// Copy `len` bytes with one wavefront. When source and destination agree
// modulo 16 the body moves as 16-byte vectors, kCopyUnroll per lane in flight;
// when they agree modulo 4 as dwords; otherwise byte by byte.
__device__ __forceinline__ void wave_copy(const char* __restrict__ s, char* __restrict__ d,
                                          uint64_t len, int lane)
{
    const uintptr_t sa = uintptr_t(s), da = uintptr_t(d);
    if (((sa ^ da) & 15) == 0) {
        uint64_t head = (16 - (da & 15)) & 15;
        if (head > len) head = len;
        if (uint64_t(lane) < head) d[lane] = s[lane];
        s += head;
        d += head;
        len -= head;
        const uint64_t nv = len >> 4;
        const V16* sv = reinterpret_cast<const V16*>(s);
        V16* dv = reinterpret_cast<V16*>(d);
        for (uint64_t base = lane; base < nv; base += 64 * kCopyUnroll) {
            V16 v[kCopyUnroll];
#pragma unroll
            for (int k = 0; k < kCopyUnroll; ++k) {
                const uint64_t i = base + 64 * k;
                if (i < nv) v[k] = ld(sv + i);
            }
#pragma unroll
            for (int k = 0; k < kCopyUnroll; ++k) {
                const uint64_t i = base + 64 * k;
                if (i < nv) st(dv + i, v[k]);
            }
        }
        const uint64_t done = nv << 4;
        if (uint64_t(lane) < len - done) d[done + lane] = s[done + lane];
    } else if (((sa ^ da) & 3) == 0) {
        uint64_t head = (4 - (da & 3)) & 3;
        if (head > len) head = len;
        if (uint64_t(lane) < head) d[lane] = s[lane];
        s += head;
        d += head;
        len -= head;
        const uint64_t nw = len >> 2;
        const uint32_t* sw = reinterpret_cast<const uint32_t*>(s);
        uint32_t* dw = reinterpret_cast<uint32_t*>(d);
        for (uint64_t i = lane; i < nw; i += 64) dw[i] = sw[i];
        const uint64_t done = nw << 2;
        if (uint64_t(lane) < len - done) d[done + lane] = s[done + lane];
    } else {
        for (uint64_t i = lane; i < len; i += 64) d[i] = s[i];
    }
}

// Fixed grid; wavefront w copies bytes [w*Q, (w+1)*Q) of the concatenation of
// all objects (Q = total / wavefronts, rounded up to 4 KiB). It finds the
// object holding its first byte from the group prefix sums (a binary search
// over groups, then a scan across the 64 lanes of that group), then walks the
// objects in order until its share is done. An object larger than Q is split
// across wavefronts; many small objects go to one wavefront.
//
// ONE_GROUP: a list of at most 64 objects is one group, so every wavefront
// scans the group's lengths itself and takes the total from the scan; no
// metadata launch runs before the copy and no group scratch is read, and the
// first wavefront counts the invalid descriptors.
//
// When the objects average at least kLargeObject bytes and the call moves at
// least kLargeCall bytes, only the first large_waves wavefronts take shares
// (the rest exit at once). Measured on MI355X, 2 workgroups per CU instead of
// 8 move a 33.5 GB list of 128 KiB objects 5.5 % faster and one 2 GiB object
// 3-4 % faster; a 0.5 GB call loses 4 % that way, and lists of small
// objects, which are bound by walking descriptors, need every wavefront.
constexpr uint64_t kLargeObject = 64 * 1024;
constexpr uint64_t kLargeCall = uint64_t(1) << 30;
template <bool ONE_GROUP>
__global__ __launch_bounds__(kBlock) void k_bc_copy(const CopyDesc* __restrict__ descs, int64_t n,
                                                    const char* __restrict__ src,
                                                    uint64_t src_bytes, char* __restrict__ dst,
                                                    uint64_t dst_bytes,
                                                    const uint64_t* __restrict__ group_base,
                                                    int64_t ngroups, uint64_t large_waves,
                                                    unsigned long long* err)
{
    const int lane = threadIdx.x & 63;
    auto inclusive_scan = [&](unsigned long long v) {
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long y = __shfl_up(v, o);
            if (lane >= o) v += y;
        }
        return v;
    };
    unsigned long long len = 0, incl = 0;
    uint64_t total;
    if constexpr (ONE_GROUP) {
        const CopyDesc x = lane < n ? descs[lane] : CopyDesc{0, 0, 0};
        len = object_bytes(x, src_bytes, dst_bytes);
        if (blockIdx.x == 0 && threadIdx.x < 64 && len != x.nbytes) atomicAdd(err, 1ull);
        incl = inclusive_scan(len);
        total = __shfl(incl, 63);
    } else {
        total = group_base[ngroups];
    }
    const uint64_t all_waves = uint64_t(gridDim.x) * kWavesPerBlock;
    const uint64_t nwaves =
        total >= uint64_t(n) * kLargeObject && total >= kLargeCall
            ? max(uint64_t(1), min(large_waves, all_waves))
            : all_waves;
    const uint64_t w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
    uint64_t share = (total + nwaves - 1) / nwaves;
    share = (share + 4095) & ~uint64_t(4095);
    const uint64_t r0 = w * share;
    if (r0 >= total) return;
    const uint64_t r1 = min(r0 + share, total);

    // last group whose first byte is <= r0
    int64_t lo = 0;
    uint64_t rel = r0;
    if constexpr (!ONE_GROUP) {
        int64_t hi = ngroups - 1;
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (group_base[mid] <= r0) lo = mid;
            else hi = mid - 1;
        }
        const int64_t k = lo * kDescGroup + lane;
        len = k < n ? object_bytes(descs[k], src_bytes, dst_bytes) : 0;
        incl = inclusive_scan(len);
        rel = r0 - group_base[lo];
    }
    const unsigned long long excl = incl - len;
    const uint64_t owner = __ballot(excl <= rel && rel < incl);
    const int first = __ffsll((unsigned long long)owner) - 1;
    int64_t kk = lo * kDescGroup + first;
    uint64_t off = rel - __shfl(excl, first);

    uint64_t pos = r0;
    CopyDesc cur = descs[kk];
    while (pos < r1) {
        CopyDesc nxt = cur;
        if (kk + 1 < n) nxt = descs[kk + 1];
        const uint64_t clen = object_bytes(cur, src_bytes, dst_bytes);
        const uint64_t take = min(clen - off, r1 - pos);
        if (take) wave_copy(src + cur.src_off + off, dst + cur.dst_off + off, take, lane);
        pos += take;
        off = 0;
        ++kk;
        cur = nxt;
    }
}

// ---------------------------------------------------- static scratch ---
// The scratch of kvm_batch_copy_noalloc: one file-scope device array per
// GPU the library runs on, held until the process ends. Host code never uses
// the array's name as an address (on the host it is only a stand-in): each
// device's address is taken once, with that device current, by
// static_scratch() below, and the kernels receive that address as an
// ordinary pointer argument.
__device__ __align__(256) uint64_t scratch[kStaticScratchWords];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint64_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(int device, uint64_t** out)
{
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device) return hipErrorInvalidDevice;  // the caller makes `device` current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = static_cast<uint64_t*>(p);
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

// ------------------------------------------------------------- launches ---

#define KVM_UNIT_SWITCH(unit, CALL)                   \
    switch (unit) {                                   \
    case 16: CALL(16); break;                         \
    case 8: CALL(8); break;                           \
    case 4: CALL(4); break;                           \
    case 2: CALL(2); break;                           \
    default: CALL(1); break;                          \
    }

// Grid of a tile kernel: one workgroup per work item, or the budget if smaller.
// A dispatch counts its grid in work-items, as a 32-bit number, so a grid of
// 1024-thread workgroups holds at most this many. Every tile kernel walks its
// items grid-stride, so a larger item count only gives each workgroup more.
constexpr int64_t kMaxGridWgs = int64_t(0xFFFFFFFFu) / 1024;

static dim3 tile_grid(int64_t ntiles, int32_t max_wgs)
{
    const int64_t n = max_wgs > 0 ? std::min<int64_t>(ntiles, max_wgs) : ntiles;
    return dim3(uint32_t(std::min(n, kMaxGridWgs)));
}

hipError_t launch_pack(int unit, const PoolGeom& g, const char* pool, int32_t num_layers,
                       const SeqBatch& b, unsigned long long* err, int32_t max_wgs,
                       hipStream_t st)
{
    const uint32_t v = uint32_t(g.row_bytes / unit);
    const FastDiv dq = make_fastdiv(v * uint32_t(g.sides)), dv = make_fastdiv(v);
    const dim3 grid = tile_grid(b.tile0[b.n], max_wgs);
    // elements of one tile: the workgroup that holds it in about one pass
    const int64_t units = int64_t(g.block_tokens) * g.sides * v;
#define KVM_PACK_BS(U, BS)                                                                  \
    hipLaunchKernelGGL((k_pack<U, BS, kPackUnroll, kPackWaveMajor>), grid, dim3(BS), 0, st, g, pool, num_layers, b, dq, dv, err)
#define KVM_PACK(U)                                                                         \
    if (units > kPackMidUnits) KVM_PACK_BS(U, kPackBS);                                     \
    else if (units > kPackSmallUnits) KVM_PACK_BS(U, kPackMidBS);                           \
    else if (units > kPackTinyUnits) KVM_PACK_BS(U, kPackSmallBS);                          \
    else KVM_PACK_BS(U, kPackTinyBS)
    KVM_UNIT_SWITCH(unit, KVM_PACK)
#undef KVM_PACK
#undef KVM_PACK_BS
    return hipGetLastError();
}

hipError_t launch_unpack_order(const SeqBatch& b, int64_t num_blocks, uint32_t* count_scratch,
                               int32_t* order, hipStream_t st)
{
    int64_t most = 0;
    for (int32_t i = 0; i < b.n; ++i) most = std::max<int64_t>(most, b.tile0[i + 1] - b.tile0[i]);
    const int64_t keys = num_blocks + 1;
    uint32_t* cnt = count_scratch;
    uint32_t* cursor = count_scratch + keys;
    const dim3 grid(uint32_t((most + 255) / 256), uint32_t(b.n));
    hipLaunchKernelGGL(k_order_zero, dim3(uint32_t(std::min<int64_t>((keys + 255) / 256, 4096))),
                       dim3(256), 0, st, cnt, keys);
    hipLaunchKernelGGL(k_order_count, grid, dim3(256), 0, st, b, num_blocks, cnt);
    hipLaunchKernelGGL(k_exclusive_scan<uint32_t>, dim3(1), dim3(1024), 0, st, cnt, cursor, keys);
    hipLaunchKernelGGL(k_order_place, grid, dim3(256), 0, st, b, num_blocks, cursor, order);
    return hipGetLastError();
}

// Tiles per unpack or fused work item: two, unless two tiles' elements would
// not fit the 32-bit element index (tiles above 2^30 elements).
static bool two_tiles(int64_t tile_units)
{
    return 2 * tile_units <= int64_t(INT32_MAX);
}

hipError_t launch_unpack(int unit, const PoolGeom& g, char* pool, int32_t num_layers,
                         int32_t layer, const SeqBatch& b, const int32_t* order,
                         unsigned long long* err, int32_t max_wgs, hipStream_t st)
{
    (void)num_layers;
    const FastDiv dv = make_fastdiv(uint32_t(g.row_bytes / unit));
    const int64_t units = int64_t(g.block_tokens) * (g.row_bytes / unit);
    const int64_t nt = b.tile0[b.n];
    if (unit == 16 && units > kUnpackWideItem) {
        hipLaunchKernelGGL((k_unpack<16, kUnpackWideBS, kUnpackWideUnroll, kUnpackWaveMajor, 1>),
                           tile_grid(nt * g.sides, max_wgs), dim3(kUnpackWideBS), 0, st, g, pool,
                           layer, b, order, dv, err);
        return hipGetLastError();
    }
    if (two_tiles(units)) {
        const dim3 grid = tile_grid((nt + 1) / 2 * g.sides, max_wgs);
#define KVM_UNPACK_BS(U, BS)                                                                \
    hipLaunchKernelGGL((k_unpack<U, BS, kUnpackUnroll, kUnpackWaveMajor, 2>), grid, dim3(BS), 0, st, g, pool, layer, b, order, dv, err)
#define KVM_UNPACK(U)                                                                       \
    if (2 * units <= kSmallPairUnits) KVM_UNPACK_BS(U, kUnpackSmallBS);                     \
    else if (2 * units > int64_t(kUnpackBS) * kUnpackUnroll) KVM_UNPACK_BS(U, kUnpackPairBS); \
    else KVM_UNPACK_BS(U, kUnpackBS)
        KVM_UNIT_SWITCH(unit, KVM_UNPACK)
#undef KVM_UNPACK
#undef KVM_UNPACK_BS
    } else {
        const dim3 grid = tile_grid(nt * g.sides, max_wgs);
#define KVM_UNPACK(U)                                                                       \
    hipLaunchKernelGGL((k_unpack<U, kUnpackBS, kUnpackUnroll, kUnpackWaveMajor, 1>), grid, dim3(kUnpackBS), 0, st, g, pool, layer, b, order, dv, err)
        KVM_UNIT_SWITCH(unit, KVM_UNPACK)
#undef KVM_UNPACK
    }
    return hipGetLastError();
}

hipError_t launch_unpack_merge(int unit, const PoolGeom& g, char* pool, int32_t layer,
                               const LayerBatch& b, const int32_t* order,
                               unsigned long long* err, int32_t max_wgs, hipStream_t st)
{
    const FastDiv dv = make_fastdiv(uint32_t(g.row_bytes / unit));
    const int64_t units = int64_t(g.block_tokens) * (g.row_bytes / unit);
    const int64_t nt = b.tile0[b.n];
    if (unit == 16 && units > kUnpackWideItem) {
        hipLaunchKernelGGL((k_unpack_merge<16, kFusedWideBS, kFusedWideUnroll, true, 1>),
                           tile_grid(nt * g.sides, max_wgs), dim3(kFusedWideBS), 0, st, g, pool,
                           layer, b, order, dv, err);
        return hipGetLastError();
    }
    if (unit == 16 && 2 * units > int64_t(kFusedBS) * kFusedUnroll) {
        // a pair of 16-byte-unit tiles that one 768 x 4 pass does not hold
        // (Llama's 32 KiB block sides) keeps 1024 x 4: one pass, +0.4-1.1 %
        hipLaunchKernelGGL((k_unpack_merge<16, kFusedPairBS, kFusedUnroll, false, 2>),
                           tile_grid((nt + 1) / 2 * g.sides, max_wgs), dim3(kFusedPairBS), 0, st,
                           g, pool, layer, b, order, dv, err);
        return hipGetLastError();
    }
    if (two_tiles(units)) {
        const dim3 grid = tile_grid((nt + 1) / 2 * g.sides, max_wgs);
#define KVM_FUSED_BS(U, BS)                                                                 \
    hipLaunchKernelGGL((k_unpack_merge<U, BS, kFusedUnroll, false, 2>), grid, dim3(BS), 0, st, g, pool, layer, b, order, dv, err)
#define KVM_FUSED(U)                                                                        \
    if (2 * units <= kSmallPairUnits) KVM_FUSED_BS(U, kFusedSmallBS);                       \
    else KVM_FUSED_BS(U, kFusedBS)
        KVM_UNIT_SWITCH(unit, KVM_FUSED)
#undef KVM_FUSED
#undef KVM_FUSED_BS
    } else {
        const dim3 grid = tile_grid(nt * g.sides, max_wgs);
#define KVM_FUSED(U)                                                                        \
    hipLaunchKernelGGL((k_unpack_merge<U, kFusedBS, kFusedUnroll, false, 1>), grid, dim3(kFusedBS), 0, st, g, pool, layer, b, order, dv, err)
        KVM_UNIT_SWITCH(unit, KVM_FUSED)
#undef KVM_FUSED
    }
    return hipGetLastError();
}

hipError_t launch_merge(int unit, int64_t row_bytes, int32_t rows_per_tile, const MergeBatch& b,
                        bool wide, int32_t max_wgs, hipStream_t st)
{
    const FastDiv dv = make_fastdiv(uint32_t(row_bytes / unit));
    const dim3 grid = tile_grid(b.tile0[b.n], max_wgs);
    if (wide && unit == 16) {
        hipLaunchKernelGGL((k_merge<16, kMergeBS, kMergeWideUnroll, kMergeWaveMajor>), grid,
                           dim3(kMergeBS), 0, st, rows_per_tile, b, dv);
        return hipGetLastError();
    }
#define KVM_MERGE(U)                                                                        \
    hipLaunchKernelGGL((k_merge<U, kMergeBS, kMergeUnroll, kMergeWaveMajor>), grid, dim3(kMergeBS), 0, st, rows_per_tile, b, dv)
    KVM_UNIT_SWITCH(unit, KVM_MERGE)
#undef KVM_MERGE
    return hipGetLastError();
}

hipError_t launch_batch_copy(char* dst, uint64_t dst_bytes, const char* src, uint64_t src_bytes,
                             const CopyDesc* descs, int64_t n, uint64_t* group_sum,
                             uint64_t* group_base, int32_t copy_blocks, int32_t large_blocks,
                             unsigned long long* err, hipStream_t st)
{
    const int64_t ng = (n + kDescGroup - 1) / kDescGroup;
    const uint64_t large_waves = uint64_t(large_blocks) * kWavesPerBlock;
    if (ng == 1) {
        hipLaunchKernelGGL(k_bc_copy<true>, dim3(uint32_t(copy_blocks)), dim3(kBlock), 0, st, descs,
                           n, src, src_bytes, dst, dst_bytes, nullptr, ng, large_waves, err);
        return hipGetLastError();
    }
    if (ng <= kSmallGroups) {
        hipLaunchKernelGGL(k_bc_sums_scan, dim3(1), dim3(1024), 0, st, descs, n, src_bytes,
                           dst_bytes, group_base, ng, err);
        hipLaunchKernelGGL(k_bc_copy<false>, dim3(uint32_t(copy_blocks)), dim3(kBlock), 0, st, descs,
                           n, src, src_bytes, dst, dst_bytes, group_base, ng, large_waves, err);
        return hipGetLastError();
    }
    const uint32_t sum_blocks = uint32_t((ng + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL(k_bc_group_sums, dim3(sum_blocks), dim3(kBlock), 0, st, descs, n,
                       src_bytes, dst_bytes, group_sum, ng, err);
    hipLaunchKernelGGL(k_exclusive_scan<unsigned long long>, dim3(1), dim3(1024), 0, st,
                       reinterpret_cast<const unsigned long long*>(group_sum),
                       reinterpret_cast<unsigned long long*>(group_base), ng);
    hipLaunchKernelGGL(k_bc_copy<false>, dim3(uint32_t(copy_blocks)), dim3(kBlock), 0, st, descs, n,
                       src, src_bytes, dst, dst_bytes, group_base, ng, large_waves, err);
    return hipGetLastError();
}

}  // namespace kvm
