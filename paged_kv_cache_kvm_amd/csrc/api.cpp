// api.cpp -- the extern "C" boundary of libkvmove: argument validation,
// per-launch record batches (passed to the kernels by value), grid sizing and
// status mapping. Every check runs before anything is enqueued, so a call that
// returns an error has no side effect.
#include "kvm.h"
#include "kvm_internal.h"

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

using kvm::CopyDesc;
using kvm::MergeRec;
using kvm::PoolGeom;
using kvm::SeqRec;

static_assert(sizeof(kvm_copy_desc) == 24, "kvm_copy_desc is 24 bytes");
static_assert(sizeof(CopyDesc) == sizeof(kvm_copy_desc), "device descriptor mirrors the ABI");
// the static scratch holds a list's group sums and bases (4 words per group + 2)
static_assert(kvm::copy_group_words(KVM_NOALLOC_MAX_DESCS) <= kvm::kStaticScratchWords,
              "kvm_batch_copy_noalloc's limit fits the static scratch");

namespace {

constexpr int64_t kMaxSeqs = int64_t(1) << 20;
constexpr int64_t kMaxTiles = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxDescs = int64_t(1) << 32;
// Merge tiles, rows per tile = max(1, tile bytes / row_bytes), all measured
// on MI355X in one process on the same buffers:
//  - rows of at least kMergeShortRow bytes: 64 KiB tiles, and a grid capped
//    at kMergeWgsPerCu workgroups per CU, each walking several tiles. On the
//    Llama layer loop (4 KiB rows, 16,640 tiles) the cap moves 6.7 % more
//    than one workgroup per tile, with a much tighter spread; 32 or 48 KiB
//    tiles change nothing. Pack and unpack lose under any cap, so they keep
//    one workgroup per tile. What holds merge there (5.6-6.2 TB/s) is the
//    read of one layer of the Full Block, 4 KiB rows at a power-of-two
//    128 KiB stride: with the same rows contiguous, or the stride padded by
//    4 KiB, one workgroup per 128 KiB tile moves 6.0-6.1 TB/s, while on the
//    strided slice no tile shape tried beats this one.
//  - shorter rows: 50 KiB tiles (44 MLA rows of 1152 B) and one workgroup
//    per tile. On the MLA loop: 6.31 TB/s, against 5.96 with 128 KiB tiles
//    and 5.57 with 128 KiB tiles under the cap; with 1024-byte rows, or 32
//    instead of 61 layers, the same choice gains 8-9 %. The tile size is
//    not smooth in effect (56 rows: 5.91, 64 rows: 6.06 TB/s): 42 to 48
//    rows are the good range in every geometry tried.
constexpr int64_t kMergeTileBytes = 64 * 1024;
constexpr int64_t kMergeShortTileBytes = 50 * 1024;
constexpr int64_t kMergeShortRow = 2048;
constexpr int32_t kMergeWgsPerCu = 16;

// Unpack tile orders (tiles sorted by destination block), one per distinct
// launch batch, kept so that a per-layer loop sorts once. The key is the
// batch's record bytes plus the pool's block count. A stale order (tables
// rewritten in place under the same pointers) is still a permutation of the
// same tiles, so results stay correct; only the write order is no longer
// ascending.
constexpr int kOrderSlots = 16;

// The latest unpack or fused launch on one stream that read a slot's order.
struct OrderReader {
    hipStream_t stream = nullptr;
    hipEvent_t done = nullptr;
};
constexpr size_t kOrderReaders = 8;  // streams tracked per slot

struct OrderSlot {
    uint64_t hash = 0;                  // of key (see order_hash)
    std::vector<char> key;
    int32_t* order = nullptr;
    int64_t cap = 0;
    hipEvent_t ready = nullptr;         // after the sort kernels
    bool ready_set = false;             // ready recorded for this sort (several streams seen)
    std::vector<OrderReader> readers;   // per stream; an eviction waits for all
    hipStream_t stream = nullptr;       // where the sort ran
    uint64_t used = 0;
    bool valid = false;
};

// The shape of a batched-copy list as the host sees it. Calls with equal keys
// (a per-layer loop, a repeated list) share one measured piece count.
struct CopyHintKey {
    int64_t n = -1;
    uintptr_t dst = 0, src = 0;
    uint64_t dst_bytes = 0, src_bytes = 0;
    uint64_t used = 0;
    bool operator==(const CopyHintKey& o) const
    {
        return n == o.n && dst == o.dst && src == o.src && dst_bytes == o.dst_bytes &&
               src_bytes == o.src_bytes;
    }
};
constexpr int kCopyHints = 64;
// Piece count assumed for a list shape seen for the first time (each
// workgroup of the copy then loops over pieces b, b + grid, ...).
constexpr int64_t kPieceGuess = 16384;
// Most pieces the allocating entry point keeps records for (192 MiB); a list
// whose piece bound is larger sends every object to the wavefront shares.
constexpr int64_t kMaxPieces = int64_t(1) << 23;
// The largest copy grid: a dispatch counts its work-items in 32 bits.
constexpr int64_t kMaxCopyGrid = int64_t(0xFFFFFFFFu) / 1024;

// Launch batches of one call, kept in the context and reused: once they have
// grown to a call's size, the call allocates no host memory. add() starts an
// empty batch (n = 0, tile0[0] = 0); records past n are stale and never read.
template <class B>
class PlanVec {
  public:
    void clear() { n_ = 0; }
    B& add()
    {
        if (n_ == v_.size()) v_.emplace_back();
        B& b = v_[n_++];
        b.n = 0;
        b.tile0[0] = 0;
        return b;
    }
    bool empty() const { return n_ == 0; }
    size_t size() const { return n_; }
    B& back() { return v_[n_ - 1]; }
    B& operator[](size_t i) { return v_[i]; }
    const B& operator[](size_t i) const { return v_[i]; }
    const B* begin() const { return v_.data(); }
    const B* end() const { return v_.data() + n_; }

  private:
    std::vector<B> v_;
    size_t n_ = 0;
};

struct SingleStream {
    hipStream_t home = nullptr;
    bool seen = false;
    bool multi = false;  // a second stream has been seen
};

}  // namespace

struct kvm_ctx {
    int device = 0;
    int num_cus = 0;
    int32_t max_wgs = 0;           // workgroup budget of every move launch; 0 = none
    bool checks = false;           // host-side precondition checks before each call
    int64_t device_bytes = 0;      // device memory held by this context
    unsigned long long* d_err = nullptr;
    uint64_t* d_copy = nullptr;    // batched-copy scratch: group sums and bases, piece records
    int64_t copy_words = 0;        // 64-bit words it holds
    // Piece counts measured by earlier copies, per list shape (see copy_grid):
    // hint_keys on the host, the counts (+ 1; 0 = not yet known) in pinned
    // host memory the kernels write.
    CopyHintKey hint_keys[kCopyHints];
    uint64_t* h_hints = nullptr;   // pinned host, kCopyHints words
    uint64_t* d_hints = nullptr;   // its device-visible address
    uint64_t hint_tick = 0;
    // The group scratch is reused by every batch copy: a call on another stream
    // first waits (on the device) for the previous call's kernels.
    hipEvent_t copy_done = nullptr;
    hipStream_t copy_stream = nullptr;
    bool copy_pending = false;
    OrderSlot orders[kOrderSlots];
    uint64_t order_tick = 0;
    // Streams seen by calls that read a cached order, and by batch copies that
    // use the group scratch. While a context has seen one stream, stream order
    // alone keeps a buffer from being rewritten under a launch that reads it,
    // so no event is recorded per call: each such record left the GPU idle
    // about 6 us between launches on MI355X. The first call on a second stream
    // retires the buffers the first stream's launches may read (enter_stream)
    // instead of waiting; from then on every call records its event.
    SingleStream order_streams;
    SingleStream copy_streams;
    uint32_t* d_count = nullptr;   // counting-sort scratch, 2 * (blocks + 2) words
    int64_t count_cap = 0;
    hipEvent_t count_done = nullptr;
    hipStream_t count_stream = nullptr;
    bool count_pending = false;
    uint64_t* static_scratch = nullptr;  // this device's static scratch (kvm_batch_copy_noalloc)
    // Scratch that launches may still read when the library replaces it (a
    // grown buffer; the scratch of the first stream when a second one comes):
    // kept, and counted in device_bytes, until the next call that
    // synchronises the device anyway (kvm_ctx_reserve, kvm_ctx_reserve_unpack,
    // kvm_take_device_errors, kvm_destroy), so that no move call waits for
    // the whole device.
    std::vector<std::pair<void*, size_t>> retired;  // pointer, bytes
    PlanVec<kvm::SeqBatch> seq_plan;       // pack and unpack
    PlanVec<kvm::LayerBatch> layer_plan;   // the fused call's hit rows
    PlanVec<kvm::SeqBatch> key_plan;       // ... and their unpack-order keys
    PlanVec<kvm::MergeBatch> merge_plan;   // merge, and the fused call's miss rows
    std::string last_error;
};

namespace {

class DeviceGuard {
  public:
    explicit DeviceGuard(int dev)
    {
        ok_ = hipGetDevice(&prev_) == hipSuccess;
        if (ok_ && prev_ != dev) ok_ = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard()
    {
        int cur = -1;
        if (hipGetDevice(&cur) == hipSuccess && cur != prev_) (void)hipSetDevice(prev_);
    }
    bool ok() const { return ok_; }

  private:
    int prev_ = 0;
    bool ok_ = false;
};

int fail_hip(kvm_ctx* ctx, hipError_t e, const char* what)
{
    if (ctx) ctx->last_error = std::string(what) + ": " + hipGetErrorString(e);
    return KVM_EHIP;
}

// Every device allocation of a context goes through these two, so that
// kvm_ctx_device_bytes can report what the context holds.
template <class T>
bool dev_alloc(kvm_ctx* c, T** p, size_t count)
{
    if (hipMalloc(reinterpret_cast<void**>(p), count * sizeof(T)) != hipSuccess) {
        *p = nullptr;
        return false;
    }
    c->device_bytes += int64_t(count * sizeof(T));
    return true;
}

template <class T>
void dev_free(kvm_ctx* c, T*& p, size_t count)
{
    if (!p) return;
    (void)hipFree(p);
    c->device_bytes -= int64_t(count * sizeof(T));
    p = nullptr;
}

// Give up a buffer that launches already enqueued may still read: it stays
// allocated (and counted) until free_retired.
template <class T>
void dev_retire(kvm_ctx* c, T*& p, size_t count)
{
    if (!p) return;
    c->retired.emplace_back(static_cast<void*>(p), count * sizeof(T));
    p = nullptr;
}

// Only after a device synchronisation.
void free_retired(kvm_ctx* c)
{
    for (const auto& r : c->retired) {
        (void)hipFree(r.first);
        c->device_bytes -= int64_t(r.second);
    }
    c->retired.clear();
}

// Widest move unit (16, 8, 4, 2, 1 bytes) that divides every value OR-ed in.
int move_unit(uint64_t bits)
{
    if ((bits & 15) == 0) return 16;
    if ((bits & 7) == 0) return 8;
    if ((bits & 3) == 0) return 4;
    if ((bits & 1) == 0) return 2;
    return 1;
}

int check_layout(const kvm_pool_layout* p, int32_t num_layers)
{
    if (!p || num_layers < 1) return KVM_EINVAL;
    if (p->num_sides < 1 || p->block_tokens < 1 || p->row_bytes < 1 || p->num_blocks < 1)
        return KVM_EINVAL;
    if (p->block_stride < 0 || p->side_stride < 0 || p->layer_stride < 0) return KVM_EINVAL;
    if (p->num_blocks > 1 && p->block_stride < int64_t(p->block_tokens) * p->row_bytes)
        return KVM_EINVAL;
    if (p->num_blocks > (int64_t(1) << 31)) return KVM_ERANGE;
    // one tile's elements are indexed in 32 bits
    const double tile = double(p->block_tokens) * p->num_sides * double(p->row_bytes);
    if (tile > double(INT32_MAX)) return KVM_ERANGE;
    return KVM_OK;
}

PoolGeom geom_of(const kvm_pool_layout* p)
{
    PoolGeom g;
    g.sides = p->num_sides;
    g.block_tokens = p->block_tokens;
    g.row_bytes = p->row_bytes;
    g.block_stride = p->block_stride;
    g.side_stride = p->side_stride;
    g.layer_stride = p->layer_stride;
    g.num_blocks = p->num_blocks;
    return g;
}

// The sequences of one call that own at least one tile, with their tile
// counts, split into launch batches of at most kvm::kRecsPerLaunch (into
// `batches`, which it clears first); *align_bits ORs their pointers and
// strides.
int plan_seqs(const kvm_pool_layout* p, int32_t num_layers, const kvm_seq* seqs, int32_t n,
              bool per_layer_tiles, PlanVec<kvm::SeqBatch>& batches, uint64_t* align_bits)
{
    batches.clear();
    if (n < 0) return KVM_EINVAL;
    if (n > 0 && !seqs) return KVM_EINVAL;
    if (n > kMaxSeqs) return KVM_ERANGE;
    const int64_t dense = int64_t(num_layers) * p->num_sides * p->row_bytes;
    uint64_t bits = 0;
    for (int32_t i = 0; i < n; ++i) {
        const kvm_seq& s = seqs[i];
        if (s.num_tokens < 0 || s.token_stride < 0) return KVM_EINVAL;
        if (s.num_tokens == 0) continue;
        if (!s.block_table || !s.full) return KVM_EINVAL;
        const int64_t ts = s.token_stride ? s.token_stride : dense;
        if (ts < dense) return KVM_EINVAL;
        const int64_t nb = (s.num_tokens + p->block_tokens - 1) / p->block_tokens;
        const int64_t tiles = per_layer_tiles ? nb * num_layers : nb;
        if (batches.empty() || batches.back().n == kvm::kRecsPerLaunch) batches.add();
        kvm::SeqBatch& b = batches.back();
        // unpack launches at most one work item per (tile, side)
        const int64_t items_per_tile = per_layer_tiles ? 1 : p->num_sides;
        if ((b.tile0[b.n] + tiles) * items_per_tile > kMaxTiles) return KVM_ERANGE;
        b.rec[b.n].block_table = s.block_table;
        b.rec[b.n].full = static_cast<const char*>(s.full);
        b.rec[b.n].num_tokens = s.num_tokens;
        b.rec[b.n].token_stride = ts;
        b.tile0[b.n + 1] = b.tile0[b.n] + tiles;
        ++b.n;
        bits |= uint64_t(uintptr_t(s.full)) | uint64_t(ts);
    }
    *align_bits = bits;
    return KVM_OK;
}

void order_release(kvm_ctx* c)
{
    for (OrderSlot& o : c->orders) {
        dev_free(c, o.order, size_t(o.cap));
        if (o.ready) (void)hipEventDestroy(o.ready);
        for (OrderReader& r : o.readers) (void)hipEventDestroy(r.done);
        o = OrderSlot();
    }
    dev_free(c, c->d_count, size_t(c->count_cap));
    if (c->count_done) (void)hipEventDestroy(c->count_done);
    c->count_cap = 0;
    c->count_done = nullptr;
}

// The key of an unpack order: the pool's block count, then the batch's first
// tiles and records, byte for byte. A lookup compares a 64-bit hash of it
// first and the bytes only where the hash matches; the key is never built.
size_t key_bytes(const kvm::SeqBatch& b)
{
    return sizeof(int64_t) * (size_t(b.n) + 2) + sizeof(kvm::SeqRec) * size_t(b.n);
}

uint64_t mix_words(uint64_t h, const void* p, size_t bytes)  // bytes: a multiple of 8
{
    const unsigned char* q = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < bytes; i += 8) {
        uint64_t w;
        std::memcpy(&w, q + i, 8);
        h = (h ^ w) * 0x9E3779B97F4A7C15ull;
        h ^= h >> 29;
    }
    return h;
}

uint64_t order_hash(const kvm::SeqBatch& b, int64_t num_blocks)
{
    static_assert(sizeof(kvm::SeqRec) % 8 == 0, "records hash as 64-bit words");
    uint64_t h = mix_words(0x243F6A8885A308D3ull, &num_blocks, sizeof(int64_t));
    h = mix_words(h, b.tile0, sizeof(int64_t) * (size_t(b.n) + 1));
    return mix_words(h, b.rec, sizeof(kvm::SeqRec) * size_t(b.n));
}

bool key_equals(const std::vector<char>& k, const kvm::SeqBatch& b, int64_t num_blocks)
{
    if (k.size() != key_bytes(b)) return false;
    const char* p = k.data();
    return std::memcmp(p, &num_blocks, sizeof(int64_t)) == 0 &&
           std::memcmp(p + sizeof(int64_t), b.tile0, sizeof(int64_t) * (size_t(b.n) + 1)) == 0 &&
           std::memcmp(p + sizeof(int64_t) * (size_t(b.n) + 2), b.rec,
                       sizeof(kvm::SeqRec) * size_t(b.n)) == 0;
}

void key_store(std::vector<char>& k, const kvm::SeqBatch& b, int64_t num_blocks)
{
    k.resize(key_bytes(b));  // keeps its capacity
    char* p = k.data();
    std::memcpy(p, &num_blocks, sizeof(int64_t));
    std::memcpy(p + sizeof(int64_t), b.tile0, sizeof(int64_t) * (size_t(b.n) + 1));
    std::memcpy(p + sizeof(int64_t) * (size_t(b.n) + 2), b.rec, sizeof(kvm::SeqRec) * size_t(b.n));
}

// Before a call on `st` that reads a cached order or the batched-copy
// scratch. The launches on the first stream recorded no events, so at the
// first call on another stream nothing tells when they end. Rather than wait
// for the device, that call retires every buffer they may still read (the
// order arrays and the sort's counters, or the copy scratch: freed at the
// next device synchronisation) and starts on fresh ones, which it allocates;
// from then on every call records events (see note_reader, kvm_batch_copy).
void retire_order_scratch(kvm_ctx* c)
{
    for (OrderSlot& o : c->orders) {
        dev_retire(c, o.order, size_t(o.cap));
        o.cap = 0;
        o.valid = false;
    }
    dev_retire(c, c->d_count, size_t(c->count_cap));
    c->count_cap = 0;
    c->count_pending = false;
}

void retire_copy_scratch(kvm_ctx* c)
{
    dev_retire(c, c->d_copy, size_t(c->copy_words));
    c->copy_words = 0;
    c->copy_pending = false;
}

void enter_stream(kvm_ctx* c, SingleStream* m, hipStream_t st, void (*retire)(kvm_ctx*))
{
    if (m->multi) return;
    if (!m->seen) {
        m->home = st;
        m->seen = true;
        return;
    }
    if (st == m->home) return;
    retire(c);
    m->multi = true;
}

// Wait on the host until every launch that read the slot's order has run.
hipError_t wait_readers(const OrderSlot& o)
{
    for (const OrderReader& r : o.readers) {
        const hipError_t e = hipEventSynchronize(r.done);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Note that a launch just enqueued on `st` reads the slot's order. One event
// per stream: a single event would cover only the latest reader, and an
// eviction could then rewrite the order while another stream still reads it.
int note_reader(kvm_ctx* c, OrderSlot* o, hipStream_t st)
{
    if (!c->order_streams.multi) return KVM_OK;  // one stream: its order suffices
    OrderReader* r = nullptr;
    for (OrderReader& x : o->readers)
        if (x.stream == st) r = &x;
    hipError_t e = hipSuccess;
    if (!r && o->readers.size() == kOrderReaders) {
        // every tracked reader done, so any of their events may be reused
        if ((e = wait_readers(*o)) != hipSuccess) return fail_hip(c, e, "hipEventSynchronize");
        r = &o->readers[0];
        r->stream = st;
    } else if (!r) {
        OrderReader x;
        if ((e = hipEventCreateWithFlags(&x.done, hipEventDisableTiming)) != hipSuccess)
            return fail_hip(c, e, "hipEventCreateWithFlags");
        x.stream = st;
        o->readers.push_back(x);
        r = &o->readers.back();
    }
    if ((e = hipEventRecord(r->done, st)) != hipSuccess) return fail_hip(c, e, "hipEventRecord");
    return KVM_OK;
}

// The unpack order of batch b, sorting it on `st` if it is not cached.
// Device memory is obtained before anything is enqueued for this batch.
int unpack_order(kvm_ctx* c, const kvm::SeqBatch& b, int64_t num_blocks, hipStream_t st,
                 OrderSlot** out)
{
    enter_stream(c, &c->order_streams, st, retire_order_scratch);
    const uint64_t hash = order_hash(b, num_blocks);
    ++c->order_tick;
    for (OrderSlot& o : c->orders) {
        if (o.valid && o.hash == hash && key_equals(o.key, b, num_blocks)) {
            if (o.stream != st && o.ready_set) {
                hipError_t e = hipStreamWaitEvent(st, o.ready, 0);
                if (e != hipSuccess) return fail_hip(c, e, "hipStreamWaitEvent");
            }
            o.used = c->order_tick;
            *out = &o;
            return KVM_OK;
        }
    }
    OrderSlot* o = &c->orders[0];
    for (OrderSlot& x : c->orders)
        if (x.used < o->used) o = &x;
    if (o->valid) {  // its sort or launches reading it may still be in flight
        hipError_t e = o->ready_set ? hipEventSynchronize(o->ready) : hipSuccess;
        if (e == hipSuccess) e = wait_readers(*o);
        if (e != hipSuccess) return fail_hip(c, e, "hipEventSynchronize");
        o->valid = false;
    }
    const int64_t ntiles = b.tile0[b.n];
    hipError_t e;
    if (!o->ready && (e = hipEventCreateWithFlags(&o->ready, hipEventDisableTiming)) != hipSuccess) {
        o->ready = nullptr;
        return fail_hip(c, e, "hipEventCreateWithFlags");
    }
    if (o->cap < ntiles) {
        // launches on the order's own stream may still read the old array
        // (they recorded no events): retire it; sizes grow at least 2x
        const int64_t cap = std::max(ntiles, 2 * o->cap);
        dev_retire(c, o->order, size_t(o->cap));
        o->cap = 0;
        if (!dev_alloc(c, &o->order, size_t(cap))) {
            c->last_error = "hipMalloc: unpack order";
            return KVM_ENOMEM;
        }
        o->cap = cap;
    }
    const int64_t words = 2 * (num_blocks + 2);
    if (c->count_cap < words) {
        const int64_t cap = std::max(words, 2 * c->count_cap);
        dev_retire(c, c->d_count, size_t(c->count_cap));
        c->count_cap = 0;
        c->count_pending = false;
        if (!dev_alloc(c, &c->d_count, size_t(cap))) {
            c->last_error = "hipMalloc: unpack order scratch";
            return KVM_ENOMEM;
        }
        c->count_cap = cap;
    }
    if (!c->count_done &&
        (e = hipEventCreateWithFlags(&c->count_done, hipEventDisableTiming)) != hipSuccess) {
        c->count_done = nullptr;
        return fail_hip(c, e, "hipEventCreateWithFlags");
    }
    if (c->count_pending && c->count_stream != st &&
        (e = hipStreamWaitEvent(st, c->count_done, 0)) != hipSuccess)
        return fail_hip(c, e, "hipStreamWaitEvent");
    e = kvm::launch_unpack_order(b, num_blocks, c->d_count, o->order, st);
    if (e != hipSuccess) return fail_hip(c, e, "unpack order launch");
    // on one stream, stream order covers later readers and the next sort;
    // the first call on a second stream retires the arrays instead
    // (enter_stream)
    o->ready_set = c->order_streams.multi;
    if (c->order_streams.multi) {
        if ((e = hipEventRecord(o->ready, st)) != hipSuccess ||
            (e = hipEventRecord(c->count_done, st)) != hipSuccess)
            return fail_hip(c, e, "hipEventRecord");
        c->count_stream = st;
        c->count_pending = true;
    }
    key_store(o->key, b, num_blocks);
    o->hash = hash;
    o->stream = st;
    o->used = c->order_tick;
    o->valid = true;
    *out = o;
    return KVM_OK;
}

// The batched-copy scratch, grown to at least `words` (2x at least): the old
// buffer is retired, since launches enqueued earlier may still read it.
int grow_copy(kvm_ctx* c, int64_t words)
{
    if (words <= c->copy_words) return KVM_OK;
    const int64_t cap = std::max<int64_t>({words, 2 * c->copy_words, 8192});
    dev_retire(c, c->d_copy, size_t(c->copy_words));
    c->copy_words = 0;
    c->copy_pending = false;
    if (!dev_alloc(c, &c->d_copy, size_t(cap))) {
        c->last_error = "hipMalloc: batched-copy scratch";
        return KVM_ENOMEM;
    }
    c->copy_words = cap;
    return KVM_OK;
}

// Pieces to size a grid for before the shape's count is known: one per object
// (at most kPieceGuess); for a list of one object, as many as the smaller
// buffer holds. One object can fill its buffers, and calls issued back to back
// reach the device before the first has left its count: a 2 GiB object at the
// one-per-object guess (a grid of 2 workgroups per CU, each looping over 32
// pieces) moved 5.5 TB/s on MI355X against 6.1 at one workgroup per piece.
int64_t first_guess(const CopyHintKey& key)
{
    if (key.n == 1) {
        const uint64_t room = std::min(key.src_bytes, key.dst_bytes);
        return int64_t(std::min<uint64_t>((room + kvm::kPieceBytes - 1) / kvm::kPieceBytes,
                                          uint64_t(kPieceGuess)));
    }
    return std::min<int64_t>(key.n, kPieceGuess);
}

// Grid of a batched copy: one workgroup per piece of the list's big objects
// (at least 2 per CU, which the wavefront shares of the other objects need),
// within the workgroup budget. The piece count is known only on the device;
// each call's metadata pass writes it into the pinned slot of the call's list
// shape, and the next call of that shape reads it here without waiting. A
// count that is stale or not yet written only changes the grid: workgroups
// past the pieces go straight to their shares, and pieces past the grid are
// taken in turn by the workgroups there are. When the count says every
// object of the shape was one piece, the call copies one object per
// workgroup with no metadata pass (*each).
int64_t copy_grid(kvm_ctx* c, const CopyHintKey& key, bool use_pieces, uint64_t** hint,
                  bool* each)
{
    *hint = nullptr;
    *each = false;
    int64_t np = 0;
    if (use_pieces) {
        CopyHintKey* slot = nullptr;
        for (CopyHintKey& k : c->hint_keys)
            if (k == key) slot = &k;
        const int idx = [&] {
            if (slot) return int(slot - c->hint_keys);
            int lru = 0;
            for (int i = 1; i < kCopyHints; ++i)
                if (c->hint_keys[i].used < c->hint_keys[lru].used) lru = i;
            return lru;
        }();
        if (!slot) {
            c->hint_keys[idx] = key;
            reinterpret_cast<volatile uint64_t*>(c->h_hints)[idx] = 0;
        }
        c->hint_keys[idx].used = ++c->hint_tick;
        const uint64_t v = reinterpret_cast<volatile uint64_t*>(c->h_hints)[idx];
        *hint = c->d_hints + idx;
        // one workgroup per object needs a grid of every object, so no budget
        if ((v & kvm::kHintUniform) && key.n > kvm::kDescGroup && key.n <= kMaxCopyGrid &&
            (c->max_wgs == 0 || c->max_wgs >= key.n)) {
            *each = true;
            np = key.n;
        } else {
            np = v ? int64_t((v & ~kvm::kHintUniform) - 1) : first_guess(key);
        }
    }
    int64_t grid = *each ? np : std::max<int64_t>(np, 2 * int64_t(c->num_cus));
    if (c->max_wgs > 0) grid = std::min<int64_t>(grid, c->max_wgs);
    return std::max<int64_t>(1, std::min(grid, kMaxCopyGrid));
}

// ------------------------------------------------ precondition checks ---
// Debug mode (kvm_ctx_set_checks): the preconditions the kernels cannot see
// are verified on the host before anything is enqueued. The caller's stream is
// synchronised first, since the tables or descriptors may be written by work
// already on it.

int fail_check(kvm_ctx* ctx, const std::string& what)
{
    ctx->last_error = "precondition: " + what;
    return KVM_ECHECK;
}

// No valid block id appears twice among the given tables (n entries each).
// Ids outside [0, num_blocks) are not a precondition violation: the kernels
// skip and count them.
int check_unique_blocks(kvm_ctx* ctx, hipStream_t st,
                        const std::vector<std::pair<const int32_t*, int64_t>>& tables,
                        int64_t num_blocks)
{
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail_hip(ctx, e, "hipStreamSynchronize");
    std::vector<int32_t> ids;
    for (const auto& t : tables) {
        const size_t at = ids.size();
        ids.resize(at + size_t(t.second));
        e = hipMemcpy(ids.data() + at, t.first, size_t(t.second) * sizeof(int32_t),
                      hipMemcpyDefault);
        if (e != hipSuccess) return fail_hip(ctx, e, "hipMemcpy (block table check)");
    }
    ids.erase(std::remove_if(ids.begin(), ids.end(),
                             [&](int32_t v) { return v < 0 || int64_t(v) >= num_blocks; }),
              ids.end());
    std::sort(ids.begin(), ids.end());
    const auto dup = std::adjacent_find(ids.begin(), ids.end());
    if (dup != ids.end())
        return fail_check(ctx, "block id " + std::to_string(*dup) +
                                   " is written twice by one call (repeated block-table entry)");
    return KVM_OK;
}

// Copy destinations are pairwise disjoint, and disjoint from every source
// range when the two buffers overlap. Objects outside their buffer are not a
// violation (the kernels skip and count them) and are left out.
int check_copy_list(kvm_ctx* ctx, hipStream_t st, uintptr_t dst_base, uint64_t dst_bytes,
                    uintptr_t src_base, uint64_t src_bytes, const kvm_copy_desc* descs,
                    int64_t n)
{
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail_hip(ctx, e, "hipStreamSynchronize");
    std::vector<kvm_copy_desc> h(static_cast<size_t>(n));
    e = hipMemcpy(h.data(), descs, size_t(n) * sizeof(kvm_copy_desc), hipMemcpyDefault);
    if (e != hipSuccess) return fail_hip(ctx, e, "hipMemcpy (copy list check)");
    struct Range { uint64_t a, b; int64_t k; };  // absolute [a, b), descriptor index
    std::vector<Range> dst, src;
    for (int64_t k = 0; k < n; ++k) {
        const kvm_copy_desc& x = h[size_t(k)];
        if (x.nbytes == 0) continue;
        const bool ok = x.src_off <= src_bytes && x.nbytes <= src_bytes - x.src_off &&
                        x.dst_off <= dst_bytes && x.nbytes <= dst_bytes - x.dst_off;
        if (!ok) continue;
        dst.push_back({dst_base + x.dst_off, dst_base + x.dst_off + x.nbytes, k});
        src.push_back({src_base + x.src_off, src_base + x.src_off + x.nbytes, k});
    }
    auto by_start = [](const Range& p, const Range& q) { return p.a < q.a; };
    std::sort(dst.begin(), dst.end(), by_start);
    for (size_t i = 1; i < dst.size(); ++i)
        if (dst[i].a < dst[i - 1].b)
            return fail_check(ctx, "copy objects " + std::to_string(dst[i - 1].k) + " and " +
                                       std::to_string(dst[i].k) + " overlap in the destination");
    const bool buffers_overlap = dst_base < src_base + src_bytes && src_base < dst_base + dst_bytes;
    if (!buffers_overlap || dst.empty()) return KVM_OK;
    // merge the source ranges, then look each destination range up among them
    std::sort(src.begin(), src.end(), by_start);
    std::vector<Range> merged;
    for (const Range& r : src) {
        if (!merged.empty() && r.a <= merged.back().b) merged.back().b = std::max(merged.back().b, r.b);
        else merged.push_back(r);
    }
    for (const Range& d : dst) {
        auto it = std::upper_bound(merged.begin(), merged.end(), d.a,
                                   [](uint64_t v, const Range& r) { return v < r.a; });
        if (it != merged.end() && it->a < d.b)
            return fail_check(ctx, "copy object " + std::to_string(d.k) +
                                       " writes over a source range");
        if (it != merged.begin() && std::prev(it)->b > d.a)
            return fail_check(ctx, "copy object " + std::to_string(d.k) +
                                       " writes over a source range");
    }
    return KVM_OK;
}

// merge_layer records split into launch batches, with the widest move unit
// that divides every pointer and stride seen.
struct MergePlan {
    MergePlan(int64_t rb, PlanVec<kvm::MergeBatch>& store)
        : row_bytes(rb), wide(rb < kMergeShortRow),
          rows_per_tile(int32_t(std::max<int64_t>(1, (wide ? kMergeShortTileBytes : kMergeTileBytes) / rb))),
          bits(uint64_t(rb)), batches(store)
    {
        batches.clear();
    }

    int add(const void* hit, int64_t hit_stride, int64_t t_hit, const void* miss,
            int64_t miss_stride, int64_t t_miss, void* out, int64_t out_stride)
    {
        if (t_hit < 0 || t_miss < 0 || hit_stride < 0 || miss_stride < 0 || out_stride < 0)
            return KVM_EINVAL;
        if ((t_hit > 0 && !hit) || (t_miss > 0 && !miss)) return KVM_EINVAL;
        const int64_t t_all = t_hit + t_miss;
        if (t_all == 0) return KVM_OK;
        if (!out) return KVM_EINVAL;
        if (batches.empty() || batches.back().n == kvm::kRecsPerLaunch) batches.add();
        kvm::MergeBatch& b = batches.back();
        const int64_t tiles = (t_all + rows_per_tile - 1) / rows_per_tile;
        if (b.tile0[b.n] + tiles > kMaxTiles) return KVM_ERANGE;
        b.rec[b.n] = {static_cast<const char*>(hit), hit_stride, t_hit,
                      static_cast<const char*>(miss), miss_stride, t_miss,
                      static_cast<char*>(out), out_stride};
        b.tile0[b.n + 1] = b.tile0[b.n] + tiles;
        ++b.n;
        bits |= uint64_t(uintptr_t(out)) | uint64_t(out_stride);
        if (t_hit > 0) bits |= uint64_t(uintptr_t(hit)) | uint64_t(hit_stride);
        if (t_miss > 0) bits |= uint64_t(uintptr_t(miss)) | uint64_t(miss_stride);
        return KVM_OK;
    }

    int launch(kvm_ctx* ctx, hipStream_t st) const
    {
        const int unit = move_unit(bits);
        // short rows: one workgroup per tile unless a budget is set
        const int32_t cap = wide ? 0 : kMergeWgsPerCu * ctx->num_cus;
        const int32_t grid = ctx->max_wgs > 0 ? (cap ? std::min(ctx->max_wgs, cap) : ctx->max_wgs)
                                              : cap;
        for (const kvm::MergeBatch& b : batches) {
            hipError_t e = kvm::launch_merge(unit, row_bytes, rows_per_tile, b, wide, grid, st);
            if (e != hipSuccess) return fail_hip(ctx, e, "k_merge launch");
        }
        return KVM_OK;
    }

    int64_t row_bytes;
    bool wide;
    int32_t rows_per_tile;
    uint64_t bits;
    PlanVec<kvm::MergeBatch>& batches;
};

}  // namespace

extern "C" {

int kvm_version(void) { return KVM_ABI_VERSION; }

const char* kvm_strerror(int status)
{
    switch (status) {
    case KVM_OK: return "ok";
    case KVM_EINVAL: return "invalid argument";
    case KVM_ERANGE: return "argument out of range";
    case KVM_ENOMEM: return "out of memory";
    case KVM_EHIP: return "HIP runtime error";
    case KVM_ECHECK: return "precondition violated (checks on)";
    default: return "unknown status";
    }
}

int kvm_create(int device, kvm_ctx** out)
{
    if (!out || device < 0) return KVM_EINVAL;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device >= count) return KVM_EHIP;
    DeviceGuard guard(device);
    if (!guard.ok()) return KVM_EHIP;
    kvm_ctx* c = new (std::nothrow) kvm_ctx();
    if (!c) return KVM_ENOMEM;
    c->device = device;
    const char* env = std::getenv("KVM_CHECK");
    c->checks = env && std::strcmp(env, "1") == 0;
    if (hipDeviceGetAttribute(&c->num_cus, hipDeviceAttributeMultiprocessorCount, device) !=
            hipSuccess ||
        c->num_cus <= 0) {
        delete c;
        return KVM_EHIP;
    }
    if (!dev_alloc(c, &c->d_err, 1)) {
        delete c;
        return KVM_ENOMEM;
    }
    if (hipMemset(c->d_err, 0, sizeof(unsigned long long)) != hipSuccess) {
        dev_free(c, c->d_err, 1);
        delete c;
        return KVM_EHIP;
    }
    int rc = grow_copy(c, kvm::copy_group_words(65536));
    if (rc == KVM_OK) {
        void* h = nullptr;
        if (hipHostMalloc(&h, sizeof(uint64_t) * kCopyHints, hipHostMallocDefault) != hipSuccess) {
            rc = KVM_ENOMEM;
        } else {
            c->h_hints = static_cast<uint64_t*>(h);
            std::memset(h, 0, sizeof(uint64_t) * kCopyHints);
            void* d = nullptr;
            if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess) rc = KVM_EHIP;
            c->d_hints = static_cast<uint64_t*>(d);
        }
    }
    if (rc == KVM_OK && hipEventCreateWithFlags(&c->copy_done, hipEventDisableTiming) != hipSuccess) {
        c->copy_done = nullptr;
        rc = KVM_EHIP;
    }
    // the static scratch's device address, taken once per device with that
    // device current (the guard above made it current)
    if (rc == KVM_OK && kvm::static_scratch(device, &c->static_scratch) != hipSuccess) {
        c->static_scratch = nullptr;
        rc = KVM_EHIP;
    }
    if (rc != KVM_OK) {
        kvm_destroy(c);
        return rc;
    }
    *out = c;
    return KVM_OK;
}

void kvm_destroy(kvm_ctx* ctx)
{
    if (!ctx) return;
    DeviceGuard guard(ctx->device);
    (void)hipDeviceSynchronize();
    free_retired(ctx);
    order_release(ctx);
    if (ctx->copy_done) (void)hipEventDestroy(ctx->copy_done);
    if (ctx->d_copy) dev_free(ctx, ctx->d_copy, size_t(ctx->copy_words));
    if (ctx->h_hints) (void)hipHostFree(ctx->h_hints);
    dev_free(ctx, ctx->d_err, 1);
    delete ctx;
}

int kvm_ctx_reserve(kvm_ctx* ctx, int64_t max_seqs, int64_t max_descs)
{
    if (!ctx || max_seqs < 0 || max_descs < 0) return KVM_EINVAL;
    if (max_seqs > kMaxSeqs || max_descs > kMaxDescs) return KVM_ERANGE;
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    // group sums and bases, and the records of one piece per object (objects
    // of up to 128 KiB); a set-up call, so it may wait for the device and
    // free what move calls retired
    const int64_t words = kvm::copy_group_words(max_descs) + 3 * std::min(max_descs, kMaxPieces);
    if (words <= ctx->copy_words && ctx->retired.empty()) return KVM_OK;
    const hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail_hip(ctx, e, "hipDeviceSynchronize");
    free_retired(ctx);
    const int rc = grow_copy(ctx, words);
    free_retired(ctx);  // the scratch it replaced: the device is idle
    return rc;
}

int kvm_ctx_reserve_unpack(kvm_ctx* ctx, int64_t max_tiles, int64_t max_pool_blocks)
{
    if (!ctx || max_tiles < 0 || max_pool_blocks < 0) return KVM_EINVAL;
    if (max_tiles > kMaxTiles || max_pool_blocks > (int64_t(1) << 31)) return KVM_ERANGE;
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    hipError_t e = hipDeviceSynchronize();  // no order or count array may be in use
    if (e != hipSuccess) return fail_hip(ctx, e, "hipDeviceSynchronize");
    free_retired(ctx);
    for (OrderSlot& o : ctx->orders) {
        if (!o.ready && (e = hipEventCreateWithFlags(&o.ready, hipEventDisableTiming)) != hipSuccess) {
            o.ready = nullptr;
            return fail_hip(ctx, e, "hipEventCreateWithFlags");
        }
        if (o.cap < max_tiles) {
            dev_free(ctx, o.order, size_t(o.cap));
            o.cap = 0;
            o.valid = false;
            if (!dev_alloc(ctx, &o.order, size_t(max_tiles))) {
                ctx->last_error = "hipMalloc: unpack order";
                return KVM_ENOMEM;
            }
            o.cap = max_tiles;
        }
    }
    const int64_t words = 2 * (max_pool_blocks + 2);
    if (ctx->count_cap < words) {
        dev_free(ctx, ctx->d_count, size_t(ctx->count_cap));
        ctx->count_cap = 0;
        ctx->count_pending = false;
        if (!dev_alloc(ctx, &ctx->d_count, size_t(words))) {
            ctx->last_error = "hipMalloc: unpack order scratch";
            return KVM_ENOMEM;
        }
        ctx->count_cap = words;
    }
    if (!ctx->count_done &&
        (e = hipEventCreateWithFlags(&ctx->count_done, hipEventDisableTiming)) != hipSuccess) {
        ctx->count_done = nullptr;
        return fail_hip(ctx, e, "hipEventCreateWithFlags");
    }
    return KVM_OK;
}

int kvm_ctx_device_bytes(const kvm_ctx* ctx, int64_t* bytes)
{
    if (!ctx || !bytes) return KVM_EINVAL;
    *bytes = ctx->device_bytes;
    return KVM_OK;
}

int kvm_ctx_set_checks(kvm_ctx* ctx, int32_t enable)
{
    if (!ctx) return KVM_EINVAL;
    ctx->checks = enable != 0;
    return KVM_OK;
}

int kvm_ctx_set_max_workgroups(kvm_ctx* ctx, int32_t max_workgroups)
{
    if (!ctx || max_workgroups < 0) return KVM_EINVAL;
    ctx->max_wgs = max_workgroups;
    return KVM_OK;
}

const char* kvm_ctx_last_error(const kvm_ctx* ctx) { return ctx ? ctx->last_error.c_str() : ""; }

int kvm_take_device_errors(kvm_ctx* ctx, int64_t* count)
{
    if (!ctx || !count) return KVM_EINVAL;
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail_hip(ctx, e, "hipDeviceSynchronize");
    free_retired(ctx);
    unsigned long long v = 0;
    e = hipMemcpy(&v, ctx->d_err, sizeof(v), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail_hip(ctx, e, "hipMemcpy (error counter)");
    e = hipMemset(ctx->d_err, 0, sizeof(v));
    if (e != hipSuccess) return fail_hip(ctx, e, "hipMemset (error counter)");
    *count = int64_t(v);
    return KVM_OK;
}

static int pack_or_unpack(kvm_ctx* ctx, const kvm_pool_layout* layout, const void* pool,
                          int32_t num_layers, int32_t layer, bool pack, const kvm_seq* seqs,
                          int32_t n, void* stream)
{
    if (!ctx) return KVM_EINVAL;
    int rc = check_layout(layout, num_layers);
    if (rc != KVM_OK) return rc;
    if (!pack && (layer < 0 || layer >= num_layers)) return KVM_ERANGE;
    PlanVec<kvm::SeqBatch>& batches = ctx->seq_plan;
    uint64_t align_bits = 0;
    rc = plan_seqs(layout, num_layers, seqs, n, pack, batches, &align_bits);
    if (rc != KVM_OK) return rc;
    if (batches.empty()) return KVM_OK;
    if (!pool) return KVM_EINVAL;
    const uint64_t bits = align_bits | uint64_t(uintptr_t(pool)) | uint64_t(layout->row_bytes) |
                          uint64_t(layout->block_stride) | uint64_t(layout->side_stride) |
                          uint64_t(layout->layer_stride);
    const int unit = move_unit(bits);

    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (ctx->checks && !pack) {
        std::vector<std::pair<const int32_t*, int64_t>> tables;
        for (const kvm::SeqBatch& b : batches)
            for (int32_t i = 0; i < b.n; ++i)
                tables.emplace_back(b.rec[i].block_table, b.tile0[i + 1] - b.tile0[i]);
        rc = check_unique_blocks(ctx, st, tables, layout->num_blocks);
        if (rc != KVM_OK) return rc;
    }
    const PoolGeom g = geom_of(layout);
    OrderSlot* orders[kOrderSlots] = {};
    if (!pack) {
        // Each batch holds its own cache slot for the whole call, so a call may
        // have at most kOrderSlots batches. Sorting runs first, so that a
        // failure leaves the caller's memory untouched (the sort kernels write
        // only the context's own scratch). The counting sort costs O(blocks);
        // for a pool much larger than the call's tiles the tiles keep their
        // own order instead.
        if (batches.size() > size_t(kOrderSlots)) return KVM_ERANGE;
        for (size_t i = 0; i < batches.size(); ++i) {
            const int64_t ntiles = batches[i].tile0[batches[i].n];
            if (layout->num_blocks > 16 * ntiles + 65536) continue;
            rc = unpack_order(ctx, batches[i], layout->num_blocks, st, &orders[i]);
            if (rc != KVM_OK) return rc;
        }
    }
    for (size_t i = 0; i < batches.size(); ++i) {
        const kvm::SeqBatch& b = batches[i];
        hipError_t e;
        if (pack) {
            e = kvm::launch_pack(unit, g, static_cast<const char*>(pool), num_layers, b, ctx->d_err,
                                 ctx->max_wgs, st);
        } else {
            e = kvm::launch_unpack(unit, g, static_cast<char*>(const_cast<void*>(pool)), num_layers,
                                   layer, b, orders[i] ? orders[i]->order : nullptr, ctx->d_err,
                                   ctx->max_wgs, st);
        }
        if (e != hipSuccess) return fail_hip(ctx, e, pack ? "k_pack launch" : "k_unpack launch");
        if (!pack && orders[i]) {
            const int rc = note_reader(ctx, orders[i], st);
            if (rc != KVM_OK) return rc;
        }
    }
    return KVM_OK;
}

int kvm_pack_full(kvm_ctx* ctx, const kvm_pool_layout* layout, const void* pool,
                  int32_t num_layers, const kvm_seq* seqs, int32_t n, void* stream)
{
    return pack_or_unpack(ctx, layout, pool, num_layers, 0, true, seqs, n, stream);
}

int kvm_unpack_layer(kvm_ctx* ctx, const kvm_pool_layout* layout, void* pool, int32_t num_layers,
                     int32_t layer, const kvm_seq* seqs, int32_t n, void* stream)
{
    return pack_or_unpack(ctx, layout, pool, num_layers, layer, false, seqs, n, stream);
}

int kvm_merge_layer(kvm_ctx* ctx, int64_t row_bytes, const kvm_merge_seq* seqs, int32_t n,
                    void* stream)
{
    if (!ctx || row_bytes < 1 || n < 0) return KVM_EINVAL;
    if (n > 0 && !seqs) return KVM_EINVAL;
    if (n > kMaxSeqs || row_bytes > INT32_MAX) return KVM_ERANGE;
    MergePlan plan(row_bytes, ctx->merge_plan);
    for (int32_t i = 0; i < n; ++i) {
        const kvm_merge_seq& m = seqs[i];
        const int rc = plan.add(m.hit, m.hit_stride, m.t_hit, m.miss, m.miss_stride, m.t_miss,
                                m.out, m.out_stride);
        if (rc != KVM_OK) return rc;
    }
    if (plan.batches.empty()) return KVM_OK;
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    return plan.launch(ctx, static_cast<hipStream_t>(stream));
}

int kvm_unpack_merge_layer(kvm_ctx* ctx, const kvm_pool_layout* layout, void* pool,
                           int32_t num_layers, int32_t layer, const kvm_layer_seq* seqs, int32_t n,
                           void* stream)
{
    if (!ctx) return KVM_EINVAL;
    int rc = check_layout(layout, num_layers);
    if (rc != KVM_OK) return rc;
    if (layer < 0 || layer >= num_layers) return KVM_ERANGE;
    if (n < 0 || (n > 0 && !seqs)) return KVM_EINVAL;
    if (n > kMaxSeqs) return KVM_ERANGE;
    const int64_t c_kv = int64_t(layout->num_sides) * layout->row_bytes;
    if (c_kv > INT32_MAX) return KVM_ERANGE;
    const int64_t dense = int64_t(num_layers) * c_kv;
    // Every record is checked first, and the move unit of the hit rows set.
    uint64_t bits = uint64_t(uintptr_t(pool)) | uint64_t(layout->row_bytes) |
                    uint64_t(layout->block_stride) | uint64_t(layout->side_stride) |
                    uint64_t(layout->layer_stride);
    for (int32_t i = 0; i < n; ++i) {
        const kvm_layer_seq& s = seqs[i];
        if (s.t_hit < 0 || s.t_miss < 0 || s.token_stride < 0 || s.miss_stride < 0 ||
            s.out_stride < 0)
            return KVM_EINVAL;
        if (s.t_hit > 0 && (!s.block_table || !s.full)) return KVM_EINVAL;
        if (s.t_miss > 0 && !s.miss) return KVM_EINVAL;
        if (s.t_hit + s.t_miss > 0 && !s.out) return KVM_EINVAL;
        const int64_t ts = s.token_stride ? s.token_stride : dense;
        if (ts < dense) return KVM_EINVAL;
        if (s.t_hit > 0)
            bits |= uint64_t(uintptr_t(s.full)) | uint64_t(ts) | uint64_t(uintptr_t(s.out)) |
                    uint64_t(s.out_stride);
    }
    const int unit = move_unit(bits);
    // Hit rows: tiles of the fused kernel. A request's miss rows go into the
    // same launch, as its last work items, when their address and stride keep
    // that unit; otherwise (and for requests with no hit rows) into a merge
    // with no hit part.
    PlanVec<kvm::LayerBatch>& hit = ctx->layer_plan;
    PlanVec<kvm::SeqBatch>& keys = ctx->key_plan;  // the same records as an unpack call, for the tile order
    hit.clear();
    keys.clear();
    MergePlan miss(c_kv, ctx->merge_plan);
    const int64_t miss_rows = std::max<int64_t>(1, kMergeTileBytes / c_kv);
    for (int32_t i = 0; i < n; ++i) {
        const kvm_layer_seq& s = seqs[i];
        const int64_t ts = s.token_stride ? s.token_stride : dense;
        const bool fold = s.t_hit > 0 && s.t_miss > 0 &&
                          ((uint64_t(uintptr_t(s.miss)) | uint64_t(s.miss_stride)) &
                           uint64_t(unit - 1)) == 0;
        if (s.t_miss > 0 && !fold) {
            rc = miss.add(nullptr, 0, 0, s.miss, s.miss_stride, s.t_miss,
                          static_cast<char*>(s.out) + s.t_hit * s.out_stride, s.out_stride);
            if (rc != KVM_OK) return rc;
        }
        if (s.t_hit == 0) continue;
        if (hit.empty() || hit.back().n == kvm::kRecsPerLaunch) {
            kvm::LayerBatch& nb = hit.add();
            nb.miss0[0] = 0;
            nb.miss_rows = int32_t(miss_rows);
            keys.add();
        }
        kvm::LayerBatch& b = hit.back();
        kvm::SeqBatch& k = keys.back();
        const int64_t tiles = (s.t_hit + layout->block_tokens - 1) / layout->block_tokens;
        if ((b.tile0[b.n] + tiles) * layout->num_sides > kMaxTiles) return KVM_ERANGE;
        const int64_t mtiles = fold ? (s.t_miss + miss_rows - 1) / miss_rows : 0;
        if (b.miss0[b.n] + mtiles > kMaxTiles) return KVM_ERANGE;
        b.rec[b.n] = {s.block_table, static_cast<const char*>(s.full), s.t_hit, ts,
                      static_cast<char*>(s.out), s.out_stride,
                      fold ? static_cast<const char*>(s.miss) : nullptr, s.miss_stride,
                      fold ? s.t_miss : 0};
        k.rec[k.n] = {s.block_table, static_cast<const char*>(s.full), s.t_hit, ts};
        b.tile0[b.n + 1] = k.tile0[k.n + 1] = b.tile0[b.n] + tiles;
        b.miss0[b.n + 1] = b.miss0[b.n] + mtiles;
        ++b.n;
        ++k.n;
    }
    if (hit.empty() && miss.batches.empty()) return KVM_OK;
    if (!hit.empty() && !pool) return KVM_EINVAL;
    if (hit.size() > size_t(kOrderSlots)) return KVM_ERANGE;

    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (ctx->checks) {
        std::vector<std::pair<const int32_t*, int64_t>> tables;
        for (const kvm::SeqBatch& b : keys)
            for (int32_t i = 0; i < b.n; ++i)
                tables.emplace_back(b.rec[i].block_table, b.tile0[i + 1] - b.tile0[i]);
        rc = check_unique_blocks(ctx, st, tables, layout->num_blocks);
        if (rc != KVM_OK) return rc;
    }
    OrderSlot* orders[kOrderSlots] = {};
    for (size_t i = 0; i < hit.size(); ++i) {
        if (layout->num_blocks > 16 * hit[i].tile0[hit[i].n] + 65536) continue;
        rc = unpack_order(ctx, keys[i], layout->num_blocks, st, &orders[i]);
        if (rc != KVM_OK) return rc;
    }
    const PoolGeom g = geom_of(layout);
    for (size_t i = 0; i < hit.size(); ++i) {
        hipError_t e = kvm::launch_unpack_merge(unit, g, static_cast<char*>(pool), layer, hit[i],
                                                c_kv, orders[i] ? orders[i]->order : nullptr,
                                                ctx->d_err, ctx->max_wgs, st);
        if (e != hipSuccess) return fail_hip(ctx, e, "k_unpack_merge launch");
        if (orders[i]) {
            rc = note_reader(ctx, orders[i], st);
            if (rc != KVM_OK) return rc;
        }
    }
    return miss.batches.empty() ? KVM_OK : miss.launch(ctx, st);
}

int kvm_batch_copy(kvm_ctx* ctx, void* dst_base, uint64_t dst_bytes, const void* src_base,
                   uint64_t src_bytes, const kvm_copy_desc* descs, int64_t n_descs, void* stream)
{
    if (!ctx || n_descs < 0) return KVM_EINVAL;
    if (n_descs == 0) return KVM_OK;
    if (!descs || !dst_base || !src_base) return KVM_EINVAL;
    if (n_descs > kMaxDescs) return KVM_ERANGE;
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    if (ctx->checks) {
        const int rc = check_copy_list(ctx, static_cast<hipStream_t>(stream),
                                       uintptr_t(dst_base), dst_bytes, uintptr_t(src_base),
                                       src_bytes, descs, n_descs);
        if (rc != KVM_OK) return rc;
    }
    // A list of one group (at most 64 objects) is copied in one launch that
    // uses no scratch: no allocation, and no wait on another stream's use of
    // the scratch.
    const int64_t groups = (n_descs + kvm::kDescGroup - 1) / kvm::kDescGroup;
    const bool one_group = groups == 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t bound = kvm::copy_piece_bound(n_descs, dst_bytes);
    const bool use_pieces = bound <= kMaxPieces;
    const int64_t piece_cap = use_pieces ? bound : 0;
    CopyHintKey key;
    key.n = n_descs;
    key.dst = uintptr_t(dst_base);
    key.src = uintptr_t(src_base);
    key.dst_bytes = dst_bytes;
    key.src_bytes = src_bytes;
    kvm::BatchCopyArgs a;
    a.grid = copy_grid(ctx, key, use_pieces, &a.hint, &a.each);
    // one group or one workgroup per object: no scratch
    const bool scratch = !one_group && !a.each;
    if (scratch) {
        enter_stream(ctx, &ctx->copy_streams, st, retire_copy_scratch);
        const int rc = grow_copy(ctx, kvm::copy_group_words(n_descs) + 3 * piece_cap);
        if (rc != KVM_OK) return rc;
    }
    a.dst = static_cast<char*>(dst_base);
    a.dst_bytes = dst_bytes;
    a.src = static_cast<const char*>(src_base);
    a.src_bytes = src_bytes;
    a.descs = reinterpret_cast<const CopyDesc*>(descs);
    a.n = n_descs;
    a.scratch = scratch ? ctx->d_copy : nullptr;
    a.piece_cap = piece_cap;
    a.use_pieces = use_pieces ? 1u : 0u;
    a.err = ctx->d_err;
    hipError_t e;
    if (scratch && ctx->copy_pending && ctx->copy_stream != st) {
        e = hipStreamWaitEvent(st, ctx->copy_done, 0);
        if (e != hipSuccess) return fail_hip(ctx, e, "hipStreamWaitEvent");
    }
    e = kvm::launch_batch_copy(a, st);
    if (e != hipSuccess) return fail_hip(ctx, e, "batch copy launch");
    if (!scratch || !ctx->copy_streams.multi) return KVM_OK;
    e = hipEventRecord(ctx->copy_done, st);
    if (e != hipSuccess) return fail_hip(ctx, e, "hipEventRecord");
    ctx->copy_stream = st;
    ctx->copy_pending = true;
    return KVM_OK;
}

int kvm_batch_copy_noalloc(kvm_ctx* ctx, void* dst_base, uint64_t dst_bytes, const void* src_base,
                           uint64_t src_bytes, const kvm_copy_desc* descs, int64_t n_descs,
                           void* stream)
{
    if (!ctx || n_descs < 0) return KVM_EINVAL;
    if (n_descs == 0) return KVM_OK;
    if (!descs || !dst_base || !src_base) return KVM_EINVAL;
    if (n_descs > KVM_NOALLOC_MAX_DESCS) return KVM_ERANGE;
    if (!ctx->static_scratch) return KVM_EHIP;
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    // The same kernels as kvm_batch_copy, with the group sums and bases and
    // the piece records in the device's static scratch (no allocation, no
    // event, no wait on another stream: calls that overlap on one device share
    // that scratch and race). Piece records that might not fit send every
    // object to the wavefront shares instead.
    const int64_t groups = (n_descs + kvm::kDescGroup - 1) / kvm::kDescGroup;
    const int64_t free_words = kvm::kStaticScratchWords - kvm::copy_group_words(n_descs);
    const int64_t bound = kvm::copy_piece_bound(n_descs, dst_bytes);
    const bool use_pieces = bound <= free_words / 3;
    CopyHintKey key;
    key.n = n_descs;
    key.dst = uintptr_t(dst_base);
    key.src = uintptr_t(src_base);
    key.dst_bytes = dst_bytes;
    key.src_bytes = src_bytes;
    kvm::BatchCopyArgs a;
    a.dst = static_cast<char*>(dst_base);
    a.dst_bytes = dst_bytes;
    a.src = static_cast<const char*>(src_base);
    a.src_bytes = src_bytes;
    a.descs = reinterpret_cast<const CopyDesc*>(descs);
    a.n = n_descs;
    a.scratch = groups == 1 ? nullptr : ctx->static_scratch;
    a.piece_cap = use_pieces ? bound : 0;
    a.use_pieces = use_pieces ? 1u : 0u;
    a.grid = copy_grid(ctx, key, use_pieces, &a.hint, &a.each);
    a.err = ctx->d_err;
    const hipError_t e = kvm::launch_batch_copy(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(ctx, e, "batch copy launch");
    return KVM_OK;
}

}  // extern "C"
