// kvm_internal.h -- records staged for the kernels and the launch entry points
// shared by the C-ABI layer (api.cpp) and the gfx950 kernels (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace kvm {

// Workgroup size of the batched-copy kernels: four wave64 wavefronts. (The
// tile kernels choose their own shapes in kernels.hip.)
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / 64;

// Copy objects are counted in groups of 64, one per lane of a wavefront.
constexpr int kDescGroup = 64;

// n / d for 32-bit n by one multiply-high, an add and a shift (division by an
// invariant integer, Granlund and Montgomery 1994). d >= 1.
struct FastDiv {
    uint32_t d;
    uint32_t m;
    uint32_t s;
};
FastDiv make_fastdiv(uint32_t d);

struct PoolGeom {
    int32_t sides;
    int32_t block_tokens;
    int64_t row_bytes;
    int64_t block_stride;
    int64_t side_stride;
    int64_t layer_stride;
    int64_t num_blocks;
};

// Per-call records travel to the kernels by value, as kernel arguments (no
// host-to-device copy per call). A call with more than kRecsPerLaunch
// sequences is split into several launches.
constexpr int kRecsPerLaunch = 128;

// One sequence of pack/unpack.
struct SeqRec {
    const int32_t* block_table;
    const char* full;
    int64_t num_tokens;
    int64_t token_stride;
};

// One request of merge.
struct MergeRec {
    const char* hit;
    int64_t hit_stride;
    int64_t t_hit;
    const char* miss;
    int64_t miss_stride;
    int64_t t_miss;
    char* out;
    int64_t out_stride;
};

// tile0[i] is the first tile of record i, ascending from 0; tile0[n] is the
// launch's tile count. Every record owns at least one tile.
struct SeqBatch {
    static constexpr bool kHasOut = false;
    int32_t n;
    int64_t tile0[kRecsPerLaunch + 1];
    SeqRec rec[kRecsPerLaunch];
};

struct MergeBatch {
    int32_t n;
    int64_t tile0[kRecsPerLaunch + 1];
    MergeRec rec[kRecsPerLaunch];
};

// One request of the fused unpack + merge: its hit rows (num_tokens of them,
// out rows 0 ..), and the miss rows the same launch copies into out rows
// num_tokens .. (t_miss of them; 0 when they go through k_merge instead).
struct LayerRec {
    const int32_t* block_table;
    const char* full;
    int64_t num_tokens;
    int64_t token_stride;
    char* out;
    int64_t out_stride;
    const char* miss;
    int64_t miss_stride;
    int64_t t_miss;
};

// tile0: the records' first hit tiles; miss0: their first miss tiles (of
// miss_rows rows each), numbered after the launch's hit work items.
struct LayerBatch {
    static constexpr bool kHasOut = true;
    int32_t n;
    int32_t miss_rows;
    int64_t tile0[kRecsPerLaunch + 1];
    int64_t miss0[kRecsPerLaunch + 1];
    LayerRec rec[kRecsPerLaunch];
};

struct CopyDesc {
    uint64_t src_off;
    uint64_t dst_off;
    uint64_t nbytes;
};

// All launches go to `st` and return the launch status. `unit` is the move
// width in bytes (16, 8, 4, 2 or 1) that divides every address and stride.
// max_wgs > 0 caps the grid of a tile kernel (each workgroup then loops over
// work items i, i + grid, ...); 0 launches one workgroup per work item.
hipError_t launch_pack(int unit, const PoolGeom& g, const char* pool, int32_t num_layers,
                       const SeqBatch& b, unsigned long long* err, int32_t max_wgs,
                       hipStream_t st);

// Work item i is side i % sides of tiles order[G*p .. G*p + G), p = i / sides,
// with G = 2 (one tile for tiles above 2048 16-byte units). order: a
// permutation of the batch's tiles made by launch_unpack_order; null keeps
// the tiles' own order.
hipError_t launch_unpack(int unit, const PoolGeom& g, char* pool, int32_t num_layers,
                         int32_t layer, const SeqBatch& b, const int32_t* order,
                         unsigned long long* err, int32_t max_wgs, hipStream_t st);

// Hit rows of one layer into the pool slots and into the output rows, one
// read per row, then the records' miss rows into their output rows;
// `order` as for launch_unpack (made from the same tables). c_kv: bytes of
// one miss row.
hipError_t launch_unpack_merge(int unit, const PoolGeom& g, char* pool, int32_t layer,
                               const LayerBatch& b, int64_t c_kv, const int32_t* order,
                               unsigned long long* err, int32_t max_wgs, hipStream_t st);

// Sort the batch's unpack tiles by destination block id into `order`
// (b.tile0[b.n] entries). count_scratch holds 2 * (num_blocks + 2) words.
hipError_t launch_unpack_order(const SeqBatch& b, int64_t num_blocks, uint32_t* count_scratch,
                               int32_t* order, hipStream_t st);

// wide (rows under 2 KiB, tiles of about 50 KiB): 16-byte moves take 1024 x 8
// unit slots per workgroup instead of 1024 x 4, so a tile fits one pass.
hipError_t launch_merge(int unit, int64_t row_bytes, int32_t rows_per_tile, const MergeBatch& b,
                        bool wide, int32_t max_wgs, hipStream_t st);

// Batched copy: objects of at least kBigObject bytes whose source,
// destination and length are multiples of 16 bytes are cut into pieces of at
// most kPieceBytes, one 1024-thread workgroup each; all other objects are
// copied by wavefronts that share their bytes equally.
constexpr uint64_t kBigObject = 16 * 1024;
constexpr uint64_t kPieceBytes = 128 * 1024;

// Set in the count a metadata pass leaves for the host when every object of
// the list was exactly one piece.
constexpr uint64_t kHintUniform = uint64_t(1) << 63;

// One piece of a big object: absolute device addresses and its length.
struct PieceRec {
    uint64_t src;
    uint64_t dst;
    uint64_t nbytes;
};

// Scratch words a list of n objects needs, without and with its pieces: two
// sums and two bases per 64-object group (plus the two totals), then one
// three-word record per piece. A list of one group needs none.
constexpr int64_t copy_group_words(int64_t n) { return 4 * ((n + kDescGroup - 1) / kDescGroup) + 2; }

// The most pieces a list can hold when its destinations are disjoint, as they
// must be: each big object is at least kBigObject bytes inside dst_bytes, and
// its pieces are one more than its bytes / kPieceBytes at most.
inline int64_t copy_piece_bound(int64_t n, uint64_t dst_bytes)
{
    const uint64_t objs = std::min<uint64_t>(uint64_t(n), dst_bytes / kBigObject);
    return int64_t(objs + dst_bytes / kPieceBytes + 1);
}

struct BatchCopyArgs {
    char* dst;
    uint64_t dst_bytes;
    const char* src;
    uint64_t src_bytes;
    const CopyDesc* descs;
    int64_t n;
    uint64_t* scratch;     // copy_group_words(n) + 3 * piece_cap words; unused for one group
    int64_t piece_cap;     // piece records the scratch holds
    uint32_t use_pieces;   // 0: every object goes to the wavefront shares
    int64_t grid;          // 1024-thread workgroups of the copy launch
    bool each;             // one workgroup per object, no metadata launch (k_bc_each)
    uint64_t* hint;        // receives the list's piece count + 1 and kHintUniform
                           // (device-visible), or null
    unsigned long long* err;
};

// Size of the static device scratch used by kvm_batch_copy_noalloc, in
// 64-bit words (16 MiB per device).
constexpr int64_t kStaticScratchWords = int64_t(2) << 20;

// The address of the static scratch on `device`, which must be the current
// device; looked up once per device (hipGetSymbolAddress) and kept.
hipError_t static_scratch(int device, uint64_t** out);

// Metadata launches (none for a list of one group), then the copy launch of
// a.grid workgroups: workgroup b copies pieces b, b + grid, ..., then its
// share of the other objects. A list of one object: one launch of its own, no
// metadata. With a.each: one launch, workgroup b copying object b whole (the
// grid then holds every object).
hipError_t launch_batch_copy(const BatchCopyArgs& a, hipStream_t st);

}  // namespace kvm
