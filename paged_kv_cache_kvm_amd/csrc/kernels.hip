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
//   k_bc_*              batched copy: objects of 16 KiB and more (16-byte
//                       aligned) in pieces of up to 128 KiB, one workgroup
//                       per piece; every other object in equal wavefront
//                       shares of their bytes. Per-group sums, their scan
//                       and the piece records come first (one workgroup for
//                       lists of up to 1,024 groups, none for one group);
//                       a list whose objects were all one piece last time
//                       is copied one workgroup per object (k_bc_each), a
//                       list of one object by k_bc_one.
//
// Page notation (DualPath KV Loading, key-objects table; Tutti reading notes,
// prerequisites 3 and 5): T tokens, L layers, C_KV = sides * row_bytes per
// token-layer row, B tokens per block, block table bt.
#include "kvm_internal.h"

#include <algorithm>
#include <mutex>

namespace kvm {

// 16-byte vectors each lane of a batched-copy wavefront keeps in flight when
// it walks small objects.
constexpr int kCopyUnroll = 4;

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
//
// The 16-byte store is inline assembly, which the compiler's hazard pass does
// not look into: CDNA needs wait states between a store of more than 64 bits
// and a VALU write of that store's data registers, and the compiler would
// count none for this one. The asm therefore ends with "s_nop 1" (two wait
// states). Without it, a copy loop whose registers the compiler reused right
// after the store wrote wrong bytes on MI355X.
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
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}

// The one-object batched copy's store: "nt" only, through the compiler (which
// then also keeps the wait states the store's data registers need).
typedef __attribute__((address_space(1))) V16 GlobalV16;

__device__ __forceinline__ void st_stream(V16* p, V16 v)
{
    __builtin_nontemporal_store(v, (GlobalV16*)p);
}

// s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8): every load and store
// this wavefront issued has completed.
__device__ __forceinline__ void wait_memory()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);
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
// The requests' miss rows follow as the launch's last work items (tiles of
// batch.miss_rows rows copied to the output rows after the hit rows), so that
// they fill the slots the hit items leave at the end of the launch instead
// of taking a merge launch of their own.
template <int U, int BS, int UNR, bool SPLIT, int G>
__global__ __launch_bounds__(BS) void k_unpack_merge(PoolGeom g, char* __restrict__ pool,
                                                     int32_t layer, const LayerBatch batch,
                                                     const int32_t* __restrict__ order,
                                                     FastDiv div_v, FastDiv div_c,
                                                     unsigned long long* err)
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
    // The miss rows: work items after the hit items, item m one tile of
    // batch.miss_rows rows of the record whose miss0 range holds m (out rows
    // from num_tokens on). Element j of a tile: row j / C, unit column j % C
    // (C = c_kv / U units, div_c), in thread-major order as k_merge.
    const int64_t nt = batch.tile0[batch.n];
    const int64_t hit_items = (G == 1 ? nt : (nt + G - 1) / G) * g.sides;
    const int64_t nm = batch.miss0[batch.n];
    const int64_t grid = gridDim.x;
    int64_t i = blockIdx.x;
    if (i < hit_items) i += (hit_items - i + grid - 1) / grid * grid;
    for (; i < hit_items + nm; i += grid) {
        const int64_t m = i - hit_items;
        const int32_t si = find_record(batch.miss0, batch.n, m);
        const LayerRec& s = batch.rec[si];
        const int64_t row0 = (m - batch.miss0[si]) * batch.miss_rows;
        const uint32_t rows = uint32_t(min(int64_t(batch.miss_rows), s.t_miss - row0));
        const char* src = s.miss + row0 * s.miss_stride;
        char* dst = s.out + (s.num_tokens + row0) * s.out_stride;
        copy_elements<U, BS, UNR, false>(rows * div_c.d, [&](uint32_t j, const char*& sp, char*& dp) {
            const uint32_t r = fdiv(j, div_c);
            const uint32_t c = j - r * div_c.d;
            sp = src + int64_t(r) * s.miss_stride + int64_t(c) * U;
            dp = dst + int64_t(r) * s.out_stride + int64_t(c) * U;
        });
    }
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

// Exclusive scan of in[0..n) by one 1024-thread workgroup: out[i] = sum of
// in[0..i), out[n] = the total. Thread t owns a contiguous chunk and loads it
// eight elements at a time, so that the loads of a chunk are in flight
// together (one dependent load per element cost 13 us on 6,250 elements).
template <class T>
__device__ __forceinline__ void block_exclusive_scan(const T* __restrict__ in, T* __restrict__ out,
                                                     int64_t n, T* wave_total)
{
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t per = (n + 1023) / 1024;
    const int64_t a = min(n, int64_t(tid) * per);
    const int64_t b = min(n, a + per);
    T local = 0;
    for (int64_t i = a; i < b; i += 8) {
        T v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = i + j < b ? in[i + j] : T(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) local += v[j];
    }
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
    for (int64_t i = a; i < b; i += 8) {
        T v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = i + j < b ? in[i + j] : T(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (i + j < b) out[i + j] = run;
            run += v[j];
        }
    }
    if (tid == 1023) out[n] = before + x;
    __syncthreads();  // wave_total may be reused
}

template <class T>
__global__ __launch_bounds__(1024) void k_exclusive_scan(const T* __restrict__ in,
                                                         T* __restrict__ out, int64_t n)
{
    __shared__ T wave_total[16];
    block_exclusive_scan(in, out, n, wave_total);
}

// ---------------------------------------------------------- batch copy ---
//
// A list is split in two by object:
//   - big objects (at least kBigObject bytes, source, destination and length
//     all multiples of 16 bytes) are cut into pieces of at most kPieceBytes,
//     and each piece is copied by one 1024-thread workgroup with the whole
//     piece in flight (8 vectors per thread, each wavefront 8 KiB of
//     consecutive bytes; 4 vectors and 4 KiB for pieces of at most 64 KiB),
//     so that the workgroups running together cover a compact stretch of a
//     few objects;
//   - every other object (short, or with source and destination not equally
//     aligned modulo 16) is copied by wavefronts that each take an equal share
//     of those objects' bytes and walk them.
// Metadata: per group of 64 objects, its small-object bytes and its pieces;
// both scanned; then one record {src, dst, bytes} per piece. A list of at
// most 64 objects (one group) needs none of it: its copy kernel computes the
// same from the 64 descriptors. A list of one object has a kernel of its own
// (k_bc_one: 6.1-6.2 TB/s on one 2 GiB object, see copy_window_piece).
//
// Measured on MI355X against a wavefront-share copy of the whole list (the
// earlier design here), in one process on two machines, all outputs
// identical: one 2 GiB object 5.2-5.5 -> 5.9-6.0 TB/s, 200,000 objects of
// 4-128 KiB 5.1 -> 5.7, the 256,000-object restore list 6.0-6.25 -> 6.2-6.25
// as one call and 5.2-5.3 -> 5.4-5.9 as 64 per-layer calls. A
// workgroup that loops over several pieces loses 5-10 %: its loads wait for
// its own earlier stores (one counter for both), so the grid holds one
// workgroup per piece where it can (see launch_batch_copy).

// Bytes object k contributes: its length, or 0 when it does not lie inside
// both buffers (then it is skipped everywhere).
__device__ __forceinline__ uint64_t object_bytes(const CopyDesc& x, uint64_t src_bytes,
                                                 uint64_t dst_bytes)
{
    const bool ok = x.src_off <= src_bytes && x.nbytes <= src_bytes - x.src_off &&
                    x.dst_off <= dst_bytes && x.nbytes <= dst_bytes - x.dst_off;
    return ok ? x.nbytes : 0;
}

// The word a metadata pass leaves for the host (see launch_batch_copy): the
// list's piece count + 1, with kHintUniform set when every object was one
// piece (no small bytes, as many pieces as objects).
__device__ __forceinline__ uint64_t hint_word(uint64_t pieces, uint64_t small, int64_t n,
                                              int64_t cap)
{
    const uint64_t np = min(pieces, uint64_t(cap));
    return (np + 1) | (small == 0 && np == uint64_t(n) ? kHintUniform : 0);
}

struct ObjSplit {
    uint64_t small;   // bytes copied by the wavefront shares
    uint64_t pieces;  // pieces copied by whole workgroups
};

__device__ __forceinline__ ObjSplit split_object(const CopyDesc& x, const char* src,
                                                 uint64_t src_bytes, const char* dst,
                                                 uint64_t dst_bytes, bool use_pieces)
{
    const uint64_t len = object_bytes(x, src_bytes, dst_bytes);
    const uint64_t bits =
        uint64_t(uintptr_t(src + x.src_off)) | uint64_t(uintptr_t(dst + x.dst_off)) | len;
    const bool big = use_pieces && len >= kBigObject && (bits & 15) == 0;
    ObjSplit s;
    s.small = big ? 0 : len;
    s.pieces = big ? (len + kPieceBytes - 1) / kPieceBytes : 0;
    return s;
}

// A 64-bit value the same in every lane, moved to scalar registers.
__device__ __forceinline__ unsigned long long uniform64(unsigned long long x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(x >> 32));
    return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// inclusive scan across the 64 lanes of a wavefront
__device__ __forceinline__ unsigned long long wave_scan(unsigned long long v, int lane)
{
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_up(v, o);
        if (lane >= o) v += y;
    }
    return v;
}

// One wavefront per group of 64 objects: the group's small-object bytes and
// its pieces.
__global__ __launch_bounds__(kBlock) void k_bc_sums(const CopyDesc* __restrict__ descs, int64_t n,
                                                    const char* src, uint64_t src_bytes,
                                                    const char* dst, uint64_t dst_bytes,
                                                    uint32_t use_pieces, uint64_t* __restrict__ sums,
                                                    int64_t ngroups, unsigned long long* err)
{
    const int lane = threadIdx.x & 63;
    const int64_t grp = int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (grp >= ngroups) return;
    const int64_t k = grp * kDescGroup + lane;
    unsigned long long small = 0, pieces = 0;
    if (k < n) {
        const CopyDesc x = descs[k];
        if (object_bytes(x, src_bytes, dst_bytes) != x.nbytes) atomicAdd(err, 1ull);
        const ObjSplit sp = split_object(x, src, src_bytes, dst, dst_bytes, use_pieces);
        small = sp.small;
        pieces = sp.pieces;
    }
    for (int o = 32; o > 0; o >>= 1) {
        small += __shfl_xor(small, o);
        pieces += __shfl_xor(pieces, o);
    }
    if (lane == 0) {
        sums[grp] = small;
        sums[ngroups + grp] = pieces;
    }
}

// One workgroup: exclusive scans of the two sum arrays, with the totals at
// index ngroups: base_small[g], base_pieces[g] for g <= ngroups.
__global__ __launch_bounds__(1024) void k_bc_scan2(const uint64_t* __restrict__ sums,
                                                   uint64_t* __restrict__ bases, int64_t ngroups)
{
    __shared__ unsigned long long wave_total[16];
    const unsigned long long* in = reinterpret_cast<const unsigned long long*>(sums);
    unsigned long long* out = reinterpret_cast<unsigned long long*>(bases);
    block_exclusive_scan(in, out, ngroups, wave_total);
    block_exclusive_scan(in + ngroups, out + ngroups + 1, ngroups, wave_total);
}

// The piece records of one group of 64 objects, written by one wavefront:
// piece e of the group (e < the group's pieces) belongs to the first lane
// whose inclusive piece count exceeds e. Records past `cap` are not written
// (only a list whose destinations overlap, a caller error, can reach it).
__device__ __forceinline__ void write_pieces(const CopyDesc& x, const ObjSplit& sp, int lane,
                                             const char* src, const char* dst, uint64_t first,
                                             PieceRec* __restrict__ pieces, int64_t cap)
{
    const unsigned long long incl = wave_scan(sp.pieces, lane);
    const unsigned long long excl = incl - sp.pieces;
    const unsigned long long total = __shfl(incl, 63);
    const uint64_t s0 = uint64_t(uintptr_t(src + x.src_off));
    const uint64_t d0 = uint64_t(uintptr_t(dst + x.dst_off));
    if (__ballot(sp.pieces > 1) == 0) {
        // every object of the group is one piece at most (up to 128 KiB):
        // each lane writes its own record, no search
        if (sp.pieces == 1 && first + excl < uint64_t(cap)) {
            PieceRec r;
            r.src = s0;
            r.dst = d0;
            r.nbytes = x.nbytes;
            pieces[first + excl] = r;
        }
        return;
    }
    for (unsigned long long base = 0; base < total; base += 64) {
        const unsigned long long e = base + lane;
        int lo = 0, hi = 63;  // first lane with incl > e (every lane takes part in the shuffles)
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (__shfl(incl, mid) > e) hi = mid;
            else lo = mid + 1;
        }
        const unsigned long long j = e - __shfl(excl, lo);
        const uint64_t s = __shfl(s0, lo), d = __shfl(d0, lo), len = __shfl(x.nbytes, lo);
        if (e < total && first + e < uint64_t(cap)) {
            PieceRec r;
            r.src = s + j * kPieceBytes;
            r.dst = d + j * kPieceBytes;
            r.nbytes = min(uint64_t(kPieceBytes), len - j * kPieceBytes);
            pieces[first + e] = r;
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_bc_map(const CopyDesc* __restrict__ descs, int64_t n,
                                                   const char* src, uint64_t src_bytes,
                                                   const char* dst, uint64_t dst_bytes,
                                                   const uint64_t* __restrict__ bases,
                                                   int64_t ngroups, PieceRec* __restrict__ pieces,
                                                   int64_t cap, uint64_t* hint)
{
    const int lane = threadIdx.x & 63;
    const int64_t grp = int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (blockIdx.x == 0 && threadIdx.x == 0 && hint)
        *hint = hint_word(bases[2 * ngroups + 1], bases[ngroups], n, cap);
    if (grp >= ngroups) return;
    // a group without pieces (small objects only) reads no descriptor
    const uint64_t first = bases[ngroups + 1 + grp];
    if (bases[ngroups + 2 + grp] == first) return;
    const int64_t k = grp * kDescGroup + lane;
    CopyDesc x = CopyDesc{0, 0, 0};
    if (k < n) x = descs[k];
    const ObjSplit sp = split_object(x, src, src_bytes, dst, dst_bytes, true);
    write_pieces(x, sp, lane, src, dst, first, pieces, cap);
}

// Lists of at most kSmallGroups groups: sums, scans and piece records in one
// workgroup. Wavefront w takes groups w, w + 16, ..., kMetaInFlight of them
// at once (their descriptor loads in flight together); a list of at most
// 16 * kMetaInFlight groups (4,096 objects, a per-layer call) keeps its
// descriptors in registers between the sums and the piece records. Measured
// on MI355X for 4,000 objects: 16.3 us with one group at a time.
constexpr int64_t kSmallGroups = 1024;
constexpr int kMetaInFlight = 4;
__global__ __launch_bounds__(1024) void k_bc_meta(const CopyDesc* __restrict__ descs, int64_t n,
                                                  const char* src, uint64_t src_bytes,
                                                  const char* dst, uint64_t dst_bytes,
                                                  uint32_t use_pieces, uint64_t* __restrict__ bases,
                                                  int64_t ngroups, PieceRec* __restrict__ pieces,
                                                  int64_t cap, uint64_t* hint,
                                                  unsigned long long* err)
{
    __shared__ unsigned long long s_small[kSmallGroups], s_pieces[kSmallGroups];
    __shared__ unsigned long long wave_total[2][16];
    __shared__ unsigned long long s_total_pieces;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    auto load4 = [&](int64_t g0, CopyDesc (&x)[kMetaInFlight]) {
#pragma unroll
        for (int q = 0; q < kMetaInFlight; ++q) {
            const int64_t g = g0 + 16 * q, k = g * kDescGroup + lane;
            x[q] = CopyDesc{0, 0, 0};
            if (g < ngroups && k < n) x[q] = descs[k];
        }
    };
    CopyDesc keep[kMetaInFlight];
    for (int64_t g0 = wid; g0 < ngroups; g0 += 16 * kMetaInFlight) {
        CopyDesc x[kMetaInFlight];
        load4(g0, x);
#pragma unroll
        for (int q = 0; q < kMetaInFlight; ++q) {
            const int64_t g = g0 + 16 * q;
            if (object_bytes(x[q], src_bytes, dst_bytes) != x[q].nbytes) atomicAdd(err, 1ull);
            const ObjSplit sp = split_object(x[q], src, src_bytes, dst, dst_bytes, use_pieces);
            unsigned long long small = sp.small, pc = sp.pieces;
            for (int o = 32; o > 0; o >>= 1) {
                small += __shfl_xor(small, o);
                pc += __shfl_xor(pc, o);
            }
            if (lane == 0 && g < ngroups) {
                s_small[g] = small;
                s_pieces[g] = pc;
            }
            keep[q] = x[q];
        }
    }
    __syncthreads();
    const unsigned long long v0 = tid < ngroups ? s_small[tid] : 0;
    const unsigned long long v1 = tid < ngroups ? s_pieces[tid] : 0;
    const unsigned long long x0 = wave_scan(v0, lane), x1 = wave_scan(v1, lane);
    if (lane == 63) {
        wave_total[0][wid] = x0;
        wave_total[1][wid] = x1;
    }
    __syncthreads();
    unsigned long long b0 = 0, b1 = 0;
    for (int w = 0; w < wid; ++w) {
        b0 += wave_total[0][w];
        b1 += wave_total[1][w];
    }
    if (tid < ngroups) {
        bases[tid] = b0 + x0 - v0;
        bases[ngroups + 1 + tid] = b1 + x1 - v1;
        s_pieces[tid] = b1 + x1 - v1;  // the group's first piece
    }
    if (tid == 1023) {
        bases[ngroups] = b0 + x0;
        bases[2 * ngroups + 1] = b1 + x1;
        s_total_pieces = b1 + x1;
        if (hint && use_pieces) *hint = hint_word(b1 + x1, b0 + x0, n, cap);
    }
    if (!use_pieces) return;
    __syncthreads();
    const bool kept = ngroups <= 16 * kMetaInFlight;
    for (int64_t g0 = wid; g0 < ngroups; g0 += 16 * kMetaInFlight) {
        CopyDesc x[kMetaInFlight];
        if (kept) {
#pragma unroll
            for (int q = 0; q < kMetaInFlight; ++q) x[q] = keep[q];
        } else {
            load4(g0, x);
        }
#pragma unroll
        for (int q = 0; q < kMetaInFlight; ++q) {
            const int64_t g = g0 + 16 * q;
            if (g >= ngroups) break;
            const unsigned long long end = g + 1 < ngroups ? s_pieces[g + 1] : s_total_pieces;
            if (end == s_pieces[g]) continue;  // no pieces in this group
            const ObjSplit sp = split_object(x[q], src, src_bytes, dst, dst_bytes, true);
            write_pieces(x[q], sp, lane, src, dst, s_pieces[g], pieces, cap);
        }
    }
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

// One piece by one 1024-thread workgroup: wavefront w moves bytes
// [w*8 KiB, (w+1)*8 KiB) of the piece, each lane 8 vectors 1 KiB apart
// (pieces of at most 64 KiB: [w*4 KiB, (w+1)*4 KiB), 4 vectors per lane).
__device__ __forceinline__ void copy_piece(uint64_t src, uint64_t dst, uint64_t nbytes)
{
    constexpr int kUnr = int(kPieceBytes / (16 * 1024));
    const V16* s = reinterpret_cast<const V16*>(src);
    V16* d = reinterpret_cast<V16*>(dst);
    const uint32_t nv = uint32_t(nbytes >> 4);
    // A piece of at most 64 KiB (an object of 16-64 KiB): every wavefront
    // moves 4 vectors per lane instead of half of them moving 8 (+0.9 % on
    // objects of 4-128 KiB, the same elsewhere, measured on MI355X).
    if (nv <= 1024 * 4) {
        constexpr int kU4 = 4;
        const uint32_t first4 = (threadIdx.x >> 6) * (64 * kU4) + (threadIdx.x & 63);
        for (uint32_t base = first4; base < nv + 1024 * kU4; base += 1024 * kU4) {
            V16 v[kU4];
#pragma unroll
            for (int k = 0; k < kU4; ++k) {
                const uint32_t j = base + k * 64;
                if (j < nv) v[k] = ld(s + j);
            }
#pragma unroll
            for (int k = 0; k < kU4; ++k) {
                const uint32_t j = base + k * 64;
                if (j < nv) st(d + j, v[k]);
            }
        }
        return;
    }
    const uint32_t first = (threadIdx.x >> 6) * (64 * kUnr) + (threadIdx.x & 63);
    // One pass over the piece (it is at most 1024 * kUnr vectors), written as
    // a loop whose bound the compiler cannot reduce to one trip: every
    // variant that it turns into straight-line code (a bound of nv, loads
    // clamped to the last vector) measured 10-15 % slower on MI355X, or
    // spilled registers.
    for (uint32_t base = first; base < nv + 1024 * kUnr; base += 1024 * kUnr) {
        V16 v[kUnr];
#pragma unroll
        for (int k = 0; k < kUnr; ++k) {
            const uint32_t j = base + k * 64;
            if (j < nv) v[k] = ld(s + j);
        }
#pragma unroll
        for (int k = 0; k < kUnr; ++k) {
            const uint32_t j = base + k * 64;
            if (j < nv) st(d + j, v[k]);
        }
    }
}

// A full piece of a list's only object. The workgroups running together then
// cover one contiguous window of the source and of the destination, and there
// each wavefront keeping one 16-byte-per-lane operation in flight (every load
// and store waited for before the next), with "nt" stores, moves 3-4 % more
// than copy_piece's eight loads in flight (measured on MI355X, one process,
// same buffers). Where the pieces running together belong to scattered
// objects the same loop loses 1-1.5 %, so it is used for one object only.
__device__ __forceinline__ void copy_window_piece(uint64_t src, uint64_t dst)
{
    constexpr int kUnr = int(kPieceBytes / (16 * 1024));
    const uint32_t i0 = (threadIdx.x >> 6) * (64 * kUnr) + (threadIdx.x & 63);
    const V16* s = reinterpret_cast<const V16*>(src) + i0;
    V16* d = reinterpret_cast<V16*>(dst) + i0;
    V16 v[kUnr];
#pragma unroll
    for (int k = 0; k < kUnr; ++k) {
        v[k] = ld(s + 64 * k);
        wait_memory();
    }
#pragma unroll
    for (int k = 0; k < kUnr; ++k) {
        st_stream(d + 64 * k, v[k]);
        wait_memory();
    }
}

// The copy: workgroup b first copies pieces b, b + grid, ... (normally just
// piece b: the grid is sized to the list's piece count), then its
// wavefronts take their shares of the small objects' bytes: wavefront w
// copies bytes [w*Q, (w+1)*Q) of those objects' concatenation (Q = total /
// wavefronts, rounded up to 4 KiB), finding the object that holds its first
// byte from the group bases (a binary search over groups, then a scan across
// the 64 lanes of that group) and walking the objects from there.
//
// ONE_GROUP: a list of 2 to 64 objects (one object: k_bc_one). The first
// wavefront of each
// workgroup reads the 64 descriptors and stages their addresses and
// inclusive piece counts in LDS; piece b belongs to the first object whose
// count exceeds b. Every wavefront then scans the small bytes across its
// lanes itself. No scratch is read; workgroup 0 counts the invalid
// descriptors and writes the piece count to `hint`.
//
// The launch bounds ask for 8 wavefronts per SIMD (at most 64 registers), so
// that two workgroups, 256 KiB of pieces, are in flight per CU.
template <bool ONE_GROUP>
__global__ __launch_bounds__(1024, 8) void k_bc_copy(const CopyDesc* __restrict__ descs, int64_t n,
                                                  const char* __restrict__ src, uint64_t src_bytes,
                                                  char* __restrict__ dst, uint64_t dst_bytes,
                                                  uint32_t use_pieces,
                                                  const uint64_t* __restrict__ bases,
                                                  int64_t ngroups,
                                                  const PieceRec* __restrict__ pieces, int64_t cap,
                                                  uint64_t* hint, unsigned long long* err)
{
    const int lane = threadIdx.x & 63;
    const int64_t grid = gridDim.x;
    // ---- pieces of big objects
    unsigned long long small_len = 0, small_incl = 0;
    if constexpr (ONE_GROUP) {
        // the first wavefront stages the pieces of the 64 objects in LDS
        __shared__ uint64_t s_src[kDescGroup], s_dst[kDescGroup], s_len[kDescGroup];
        __shared__ unsigned long long s_incl[kDescGroup];
        if (threadIdx.x < 64) {
            const CopyDesc x = lane < n ? descs[lane] : CopyDesc{0, 0, 0};
            if (blockIdx.x == 0 && object_bytes(x, src_bytes, dst_bytes) != x.nbytes)
                atomicAdd(err, 1ull);
            const ObjSplit sp = split_object(x, src, src_bytes, dst, dst_bytes, use_pieces);
            s_src[lane] = uint64_t(uintptr_t(src + x.src_off));
            s_dst[lane] = uint64_t(uintptr_t(dst + x.dst_off));
            s_len[lane] = x.nbytes;
            s_incl[lane] = wave_scan(sp.pieces, lane);
        }
        __syncthreads();
        const unsigned long long np = uniform64(s_incl[63]);
        if (blockIdx.x == 0 && threadIdx.x == 0 && hint && use_pieces) *hint = np + 1;
        for (unsigned long long b = blockIdx.x; b < np; b += grid) {
            int lo = 0, hi = 63;  // first object whose inclusive piece count exceeds b
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_incl[mid] > b) hi = mid;
                else lo = mid + 1;
            }
            // the same in every lane: keep them in scalar registers
            const unsigned long long j = uniform64(b - (lo ? s_incl[lo - 1] : 0));
            const uint64_t len = uniform64(s_len[lo]);
            copy_piece(uniform64(s_src[lo]) + j * kPieceBytes, uniform64(s_dst[lo]) + j * kPieceBytes,
                       min(uint64_t(kPieceBytes), len - j * kPieceBytes));
        }
        const CopyDesc x = lane < n ? descs[lane] : CopyDesc{0, 0, 0};
        small_len = split_object(x, src, src_bytes, dst, dst_bytes, use_pieces).small;
        small_incl = wave_scan(small_len, lane);
    } else if (use_pieces) {
        const uint64_t np = min(bases[2 * ngroups + 1], uint64_t(cap));
        for (uint64_t b = blockIdx.x; b < np; b += grid) {
            const PieceRec r = pieces[b];
            copy_piece(r.src, r.dst, r.nbytes);
        }
    }
    // ---- shares of the small objects
    const uint64_t total = ONE_GROUP ? uint64_t(__shfl(small_incl, 63)) : bases[ngroups];
    if (total == 0) return;
    const uint64_t nwaves = uint64_t(grid) * (1024 / 64);
    const uint64_t w = __builtin_amdgcn_readfirstlane(blockIdx.x * (1024 / 64) + (threadIdx.x >> 6));
    uint64_t share = (total + nwaves - 1) / nwaves;
    share = (share + 4095) & ~uint64_t(4095);
    const uint64_t r0 = w * share;
    if (r0 >= total) return;
    const uint64_t r1 = min(r0 + share, total);
    auto small_of = [&](const CopyDesc& x) {
        return split_object(x, src, src_bytes, dst, dst_bytes, use_pieces).small;
    };
    // last group whose first byte is <= r0
    int64_t lo = 0;
    uint64_t rel = r0;
    unsigned long long len = small_len, incl = small_incl;
    if constexpr (!ONE_GROUP) {
        int64_t hi = ngroups - 1;
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (bases[mid] <= r0) lo = mid;
            else hi = mid - 1;
        }
        const int64_t k = lo * kDescGroup + lane;
        len = k < n ? small_of(descs[k]) : 0;
        incl = wave_scan(len, lane);
        rel = r0 - bases[lo];
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
        const uint64_t clen = small_of(cur);
        const uint64_t take = min(clen - off, r1 - pos);
        if (take) wave_copy(src + cur.src_off + off, dst + cur.dst_off + off, take, lane);
        pos += take;
        off = 0;
        ++kk;
        cur = nxt;
    }
}

// A list of one object, with no staging: every workgroup reads the descriptor
// itself. A big object (as split_object) is copied piece by piece, the full
// pieces by copy_window_piece (the last, shorter one a vector per thread at a
// time); any other object in equal wavefront shares of
// its bytes (multiples of 4 KiB), as k_bc_copy copies small objects. Workgroup
// 0 counts an object outside the buffers (then nothing is copied) and leaves
// the piece count + 1 in `hint`, as the one-group launch does.
__global__ __launch_bounds__(1024, 8) void k_bc_one(const CopyDesc* __restrict__ descs,
                                                    const char* __restrict__ src,
                                                    uint64_t src_bytes, char* __restrict__ dst,
                                                    uint64_t dst_bytes, uint32_t use_pieces,
                                                    uint64_t* hint, unsigned long long* err)
{
    const CopyDesc x = descs[0];
    const uint64_t len = object_bytes(x, src_bytes, dst_bytes);
    const ObjSplit sp = split_object(x, src, src_bytes, dst, dst_bytes, use_pieces);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (len != x.nbytes) atomicAdd(err, 1ull);
        if (hint && use_pieces) *hint = sp.pieces + 1;
    }
    const uint64_t s0 = uint64_t(uintptr_t(src + x.src_off));
    const uint64_t d0 = uint64_t(uintptr_t(dst + x.dst_off));
    const uint64_t grid = gridDim.x;
    if (sp.pieces) {
        for (uint64_t b = blockIdx.x; b < sp.pieces; b += grid) {
            const uint64_t at = b * kPieceBytes;
            if (len - at >= kPieceBytes) {
                copy_window_piece(s0 + at, d0 + at);
            } else {  // the last piece, shorter: one vector per thread at a time
                const V16* sv = reinterpret_cast<const V16*>(s0 + at);
                V16* dv = reinterpret_cast<V16*>(d0 + at);
                const uint32_t nv = uint32_t((len - at) >> 4);
                for (uint32_t u = threadIdx.x; u < nv; u += 1024) st_stream(dv + u, ld(sv + u));
            }
        }
        return;
    }
    const uint64_t nwaves = grid * (1024 / 64);
    const uint64_t w = __builtin_amdgcn_readfirstlane(blockIdx.x * (1024 / 64) + (threadIdx.x >> 6));
    uint64_t share = (len + nwaves - 1) / nwaves;
    share = (share + 4095) & ~uint64_t(4095);
    const uint64_t r0 = w * share;
    if (r0 >= len) return;
    const uint64_t r1 = min(r0 + share, len);
    wave_copy(reinterpret_cast<const char*>(s0) + r0, reinterpret_cast<char*>(d0) + r0, r1 - r0,
              int(threadIdx.x & 63));
}

// One workgroup per object, straight from the descriptors (no metadata
// launch): workgroup k copies object k. A big object (as split_object) is
// copied piece by piece as copy_piece does; any other object byte by byte by
// the whole workgroup. Correct for every list; it is the launch of choice
// only when every object is one piece, which the previous call of the same
// list shape reported (hint_word). An object that is not one piece clears the
// hint, so that the next call of the shape takes the metadata path again.
__global__ __launch_bounds__(1024, 8) void k_bc_each(const CopyDesc* __restrict__ descs, int64_t n,
                                                     const char* __restrict__ src,
                                                     uint64_t src_bytes, char* __restrict__ dst,
                                                     uint64_t dst_bytes, uint64_t* hint,
                                                     unsigned long long* err)
{
    const int64_t k = blockIdx.x;
    if (k >= n) return;
    const CopyDesc x = descs[k];
    const uint64_t len = object_bytes(x, src_bytes, dst_bytes);
    const ObjSplit sp = split_object(x, src, src_bytes, dst, dst_bytes, true);
    if (threadIdx.x == 0) {
        if (len != x.nbytes) atomicAdd(err, 1ull);
        if (hint && sp.pieces != 1) *hint = 0;
    }
    if (sp.pieces == 1) {
        copy_piece(uint64_t(uintptr_t(src + x.src_off)), uint64_t(uintptr_t(dst + x.dst_off)), len);
        return;
    }
    // Not one piece: only after a list shape changed (the hint is now
    // cleared). Simple loops keep this launch lean: 16-byte vectors for a big
    // object (aligned, by split_object), bytes otherwise.
    const char* s = src + x.src_off;
    char* d = dst + x.dst_off;
    if (sp.pieces) {
        const V16* sv = reinterpret_cast<const V16*>(s);
        V16* dv = reinterpret_cast<V16*>(d);
        for (uint64_t u = threadIdx.x; u < (len >> 4); u += 1024) st(dv + u, ld(sv + u));
    } else {
        for (uint64_t i = threadIdx.x; i < len; i += 1024) d[i] = s[i];
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
                               const LayerBatch& b, int64_t c_kv, const int32_t* order,
                               unsigned long long* err, int32_t max_wgs, hipStream_t st)
{
    const FastDiv dv = make_fastdiv(uint32_t(g.row_bytes / unit));
    const FastDiv dc = make_fastdiv(uint32_t(c_kv / unit));
    const int64_t units = int64_t(g.block_tokens) * (g.row_bytes / unit);
    const int64_t nt = b.tile0[b.n];
    const int64_t nm = b.miss0[b.n];  // miss tiles, after the hit items
    if (unit == 16 && units > kUnpackWideItem) {
        hipLaunchKernelGGL((k_unpack_merge<16, kFusedWideBS, kFusedWideUnroll, true, 1>),
                           tile_grid(nt * g.sides + nm, max_wgs), dim3(kFusedWideBS), 0, st, g,
                           pool, layer, b, order, dv, dc, err);
        return hipGetLastError();
    }
    if (unit == 16 && 2 * units > int64_t(kFusedBS) * kFusedUnroll) {
        // a pair of 16-byte-unit tiles that one 768 x 4 pass does not hold
        // (Llama's 32 KiB block sides) keeps 1024 x 4: one pass, +0.4-1.1 %
        hipLaunchKernelGGL((k_unpack_merge<16, kFusedPairBS, kFusedUnroll, false, 2>),
                           tile_grid((nt + 1) / 2 * g.sides + nm, max_wgs), dim3(kFusedPairBS), 0,
                           st, g, pool, layer, b, order, dv, dc, err);
        return hipGetLastError();
    }
    if (two_tiles(units)) {
        const dim3 grid = tile_grid((nt + 1) / 2 * g.sides + nm, max_wgs);
#define KVM_FUSED_BS(U, BS)                                                                 \
    hipLaunchKernelGGL((k_unpack_merge<U, BS, kFusedUnroll, false, 2>), grid, dim3(BS), 0, st, g, pool, layer, b, order, dv, dc, err)
#define KVM_FUSED(U)                                                                        \
    if (2 * units <= kSmallPairUnits) KVM_FUSED_BS(U, kFusedSmallBS);                       \
    else KVM_FUSED_BS(U, kFusedBS)
        KVM_UNIT_SWITCH(unit, KVM_FUSED)
#undef KVM_FUSED
#undef KVM_FUSED_BS
    } else {
        const dim3 grid = tile_grid(nt * g.sides + nm, max_wgs);
#define KVM_FUSED(U)                                                                        \
    hipLaunchKernelGGL((k_unpack_merge<U, kFusedBS, kFusedUnroll, false, 1>), grid, dim3(kFusedBS), 0, st, g, pool, layer, b, order, dv, dc, err)
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

hipError_t launch_batch_copy(const BatchCopyArgs& a, hipStream_t st)
{
    const int64_t ng = (a.n + kDescGroup - 1) / kDescGroup;
    const dim3 grid(uint32_t(a.grid));
    if (a.each) {
        hipLaunchKernelGGL(k_bc_each, grid, dim3(1024), 0, st, a.descs, a.n, a.src, a.src_bytes,
                           a.dst, a.dst_bytes, a.hint, a.err);
        return hipGetLastError();
    }
    if (a.n == 1) {
        hipLaunchKernelGGL(k_bc_one, grid, dim3(1024), 0, st, a.descs, a.src, a.src_bytes, a.dst,
                           a.dst_bytes, a.use_pieces, a.hint, a.err);
        return hipGetLastError();
    }
    if (ng == 1) {
        hipLaunchKernelGGL(k_bc_copy<true>, grid, dim3(1024), 0, st, a.descs, a.n, a.src, a.src_bytes,
                           a.dst, a.dst_bytes, a.use_pieces, nullptr, ng, nullptr, int64_t(0), a.hint,
                           a.err);
        return hipGetLastError();
    }
    uint64_t* sums = a.scratch;                       // [2 * ng]
    uint64_t* bases = a.scratch + 2 * ng;             // [2 * (ng + 1)]
    PieceRec* pieces = reinterpret_cast<PieceRec*>(a.scratch + 4 * ng + 2);
    if (ng <= kSmallGroups) {
        hipLaunchKernelGGL(k_bc_meta, dim3(1), dim3(1024), 0, st, a.descs, a.n, a.src, a.src_bytes,
                           a.dst, a.dst_bytes, a.use_pieces, bases, ng, pieces, a.piece_cap, a.hint,
                           a.err);
    } else {
        const uint32_t blocks = uint32_t((ng + kWavesPerBlock - 1) / kWavesPerBlock);
        hipLaunchKernelGGL(k_bc_sums, dim3(blocks), dim3(kBlock), 0, st, a.descs, a.n, a.src,
                           a.src_bytes, a.dst, a.dst_bytes, a.use_pieces, sums, ng, a.err);
        hipLaunchKernelGGL(k_bc_scan2, dim3(1), dim3(1024), 0, st, sums, bases, ng);
        if (a.use_pieces)
            hipLaunchKernelGGL(k_bc_map, dim3(blocks), dim3(kBlock), 0, st, a.descs, a.n, a.src,
                               a.src_bytes, a.dst, a.dst_bytes, bases, ng, pieces, a.piece_cap,
                               a.hint);
    }
    hipLaunchKernelGGL(k_bc_copy<false>, grid, dim3(1024), 0, st, a.descs, a.n, a.src, a.src_bytes,
                       a.dst, a.dst_bytes, a.use_pieces, bases, ng, pieces, a.piece_cap, a.hint,
                       a.err);
    return hipGetLastError();
}

}  // namespace kvm
