// api.cpp -- the extern "C" boundary of libkvmove: argument validation,
// per-call staging of the small per-sequence records, grid sizing and status
// mapping. Every check runs before anything is enqueued, so a call that
// returns an error has no side effect.
#include "kvm.h"
#include "kvm_internal.h"

#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

using kvm::CopyDesc;
using kvm::MergeRec;
using kvm::PoolGeom;
using kvm::SeqRec;

static_assert(sizeof(kvm_copy_desc) == 24, "kvm_copy_desc is 24 bytes");
static_assert(sizeof(CopyDesc) == sizeof(kvm_copy_desc), "device descriptor mirrors the ABI");

namespace {

constexpr int64_t kMaxSeqs = int64_t(1) << 20;
constexpr int64_t kMaxTiles = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxDescs = int64_t(1) << 32;
constexpr int kStageSlots = 32;
// Target bytes per merge tile; rows per tile = max(1, this / row_bytes).
constexpr int64_t kMergeTileBytes = 64 * 1024;

// A pinned host ring and a device ring of equal slots. A call copies its
// records into a host slot and enqueues one small host-to-device copy on the
// caller's stream; an event recorded after the kernel marks when the slot may
// be overwritten. A call whose records are byte-identical to a slot staged
// earlier on the same stream reuses that slot without a copy: in a per-layer
// loop the unpack records repeat every layer. Slots are replaced least
// recently used first.
struct Stage {
    char* host = nullptr;
    char* dev = nullptr;
    size_t slot_bytes = 0;
    uint64_t tick = 0;
    hipEvent_t done[kStageSlots] = {};
    bool busy[kStageSlots] = {};
    bool valid[kStageSlots] = {};
    uint64_t used[kStageSlots] = {};
    hipStream_t stream[kStageSlots] = {};
    std::vector<char> content[kStageSlots];
};

}  // namespace

struct kvm_ctx {
    int device = 0;
    int num_cus = 0;
    Stage stage;
    unsigned long long* d_err = nullptr;
    uint64_t* d_groups = nullptr;  // group sums, then group bases
    int64_t group_cap = 0;         // groups the scratch holds
    // The group scratch is reused by every batch copy: a call on another stream
    // first waits (on the device) for the previous call's kernels.
    hipEvent_t copy_done = nullptr;
    hipStream_t copy_stream = nullptr;
    bool copy_pending = false;
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

void stage_release(kvm_ctx* c)
{
    Stage& s = c->stage;
    for (int i = 0; i < kStageSlots; ++i) {
        if (s.done[i]) {
            if (s.busy[i]) (void)hipEventSynchronize(s.done[i]);
            (void)hipEventDestroy(s.done[i]);
            s.done[i] = nullptr;
        }
        s.busy[i] = false;
    }
    if (s.host) (void)hipHostFree(s.host);
    if (s.dev) (void)hipFree(s.dev);
    s.host = nullptr;
    s.dev = nullptr;
    s.slot_bytes = 0;
    for (int i = 0; i < kStageSlots; ++i) {
        s.valid[i] = false;
        s.used[i] = 0;
        s.content[i].clear();
    }
}

int stage_reserve(kvm_ctx* c, size_t slot_bytes)
{
    slot_bytes = (slot_bytes + 4095) & ~size_t(4095);
    if (slot_bytes <= c->stage.slot_bytes) return KVM_OK;
    stage_release(c);
    Stage& s = c->stage;
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&s.host), slot_bytes * kStageSlots,
                                 hipHostMallocDefault);
    if (e != hipSuccess) {
        s.host = nullptr;
        c->last_error = std::string("hipHostMalloc: ") + hipGetErrorString(e);
        return KVM_ENOMEM;
    }
    e = hipMalloc(reinterpret_cast<void**>(&s.dev), slot_bytes * kStageSlots);
    if (e != hipSuccess) {
        s.dev = nullptr;
        stage_release(c);
        c->last_error = std::string("hipMalloc: ") + hipGetErrorString(e);
        return KVM_ENOMEM;
    }
    for (int i = 0; i < kStageSlots; ++i) {
        e = hipEventCreateWithFlags(&s.done[i], hipEventDisableTiming);
        if (e != hipSuccess) {
            s.done[i] = nullptr;
            stage_release(c);
            return fail_hip(c, e, "hipEventCreateWithFlags");
        }
    }
    s.slot_bytes = slot_bytes;
    return KVM_OK;
}

// Put `len` bytes where the next kernel on `st` can read them; *slot is the
// slot to mark once that kernel is enqueued.
int stage_put(kvm_ctx* c, const void* bytes, size_t len, hipStream_t st, char** dptr, int* slot)
{
    int rc = stage_reserve(c, len);
    if (rc != KVM_OK) return rc;
    Stage& s = c->stage;
    ++s.tick;
    for (int k = 0; k < kStageSlots; ++k) {
        if (s.valid[k] && s.stream[k] == st && s.content[k].size() == len &&
            std::memcmp(s.content[k].data(), bytes, len) == 0) {
            s.used[k] = s.tick;
            *slot = k;
            *dptr = s.dev + size_t(k) * s.slot_bytes;
            return KVM_OK;
        }
    }
    int i = 0;
    for (int k = 1; k < kStageSlots; ++k)
        if (s.used[k] < s.used[i]) i = k;
    s.valid[i] = false;
    if (s.busy[i]) {
        hipError_t e = hipEventSynchronize(s.done[i]);
        if (e != hipSuccess) return fail_hip(c, e, "hipEventSynchronize");
        s.busy[i] = false;
    }
    char* h = s.host + size_t(i) * s.slot_bytes;
    char* d = s.dev + size_t(i) * s.slot_bytes;
    std::memcpy(h, bytes, len);
    hipError_t e = hipMemcpyAsync(d, h, len, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return fail_hip(c, e, "hipMemcpyAsync (records)");
    s.content[i].assign(static_cast<const char*>(bytes), static_cast<const char*>(bytes) + len);
    s.stream[i] = st;
    s.used[i] = s.tick;
    s.valid[i] = true;
    *slot = i;
    *dptr = d;
    return KVM_OK;
}

int stage_mark(kvm_ctx* c, int slot, hipStream_t st)
{
    hipError_t e = hipEventRecord(c->stage.done[slot], st);
    if (e != hipSuccess) return fail_hip(c, e, "hipEventRecord");
    c->stage.busy[slot] = true;
    return KVM_OK;
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

// Records for pack/unpack: [tile0 array padded to 64 entries][SeqRec array].
struct SeqPlan {
    std::vector<char> bytes;
    int32_t nrec = 0;
    int64_t ntiles = 0;
    uint64_t align_bits = 0;
    size_t rec_offset = 0;
};

int plan_seqs(const kvm_pool_layout* p, int32_t num_layers, const kvm_seq* seqs, int32_t n,
              bool per_layer_tiles, SeqPlan* plan)
{
    if (n < 0) return KVM_EINVAL;
    if (n > 0 && !seqs) return KVM_EINVAL;
    if (n > kMaxSeqs) return KVM_ERANGE;
    const int64_t dense = int64_t(num_layers) * p->num_sides * p->row_bytes;
    std::vector<int64_t> tile0;
    std::vector<SeqRec> recs;
    int64_t tiles = 0;
    uint64_t bits = 0;
    for (int32_t i = 0; i < n; ++i) {
        const kvm_seq& s = seqs[i];
        if (s.num_tokens < 0 || s.token_stride < 0) return KVM_EINVAL;
        if (s.num_tokens == 0) continue;
        if (!s.block_table || !s.full) return KVM_EINVAL;
        const int64_t ts = s.token_stride ? s.token_stride : dense;
        if (ts < dense) return KVM_EINVAL;
        const int64_t nb = (s.num_tokens + p->block_tokens - 1) / p->block_tokens;
        const int64_t t = per_layer_tiles ? nb * num_layers : nb;
        tile0.push_back(tiles);
        tiles += t;
        if (tiles > kMaxTiles) return KVM_ERANGE;
        SeqRec r;
        r.block_table = s.block_table;
        r.full = static_cast<const char*>(s.full);
        r.num_tokens = s.num_tokens;
        r.token_stride = ts;
        recs.push_back(r);
        bits |= uint64_t(uintptr_t(s.full)) | uint64_t(ts);
    }
    plan->nrec = int32_t(recs.size());
    plan->ntiles = tiles;
    plan->align_bits = bits;
    const size_t padded = (tile0.size() + 63) / 64 * 64;
    plan->rec_offset = padded * sizeof(int64_t);
    plan->bytes.assign(plan->rec_offset + recs.size() * sizeof(SeqRec), 0);
    if (!tile0.empty()) std::memcpy(plan->bytes.data(), tile0.data(), tile0.size() * sizeof(int64_t));
    if (!recs.empty())
        std::memcpy(plan->bytes.data() + plan->rec_offset, recs.data(), recs.size() * sizeof(SeqRec));
    return KVM_OK;
}

int grow_groups(kvm_ctx* c, int64_t groups)
{
    if (groups <= c->group_cap) return KVM_OK;
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail_hip(c, e, "hipDeviceSynchronize");
    if (c->d_groups) (void)hipFree(c->d_groups);
    c->d_groups = nullptr;
    c->group_cap = 0;
    const int64_t cap = std::max<int64_t>(groups, 1024);
    e = hipMalloc(reinterpret_cast<void**>(&c->d_groups), size_t(2 * cap + 1) * sizeof(uint64_t));
    if (e != hipSuccess) {
        c->d_groups = nullptr;
        c->last_error = std::string("hipMalloc: ") + hipGetErrorString(e);
        return KVM_ENOMEM;
    }
    c->group_cap = cap;
    return KVM_OK;
}

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
    if (hipDeviceGetAttribute(&c->num_cus, hipDeviceAttributeMultiprocessorCount, device) !=
            hipSuccess ||
        c->num_cus <= 0) {
        delete c;
        return KVM_EHIP;
    }
    if (hipMalloc(reinterpret_cast<void**>(&c->d_err), sizeof(unsigned long long)) != hipSuccess) {
        delete c;
        return KVM_ENOMEM;
    }
    if (hipMemset(c->d_err, 0, sizeof(unsigned long long)) != hipSuccess) {
        (void)hipFree(c->d_err);
        delete c;
        return KVM_EHIP;
    }
    int rc = stage_reserve(c, 64 * 1024);
    if (rc == KVM_OK) rc = grow_groups(c, 1024);
    if (rc == KVM_OK && hipEventCreateWithFlags(&c->copy_done, hipEventDisableTiming) != hipSuccess) {
        c->copy_done = nullptr;
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
    stage_release(ctx);
    (void)hipDeviceSynchronize();
    if (ctx->copy_done) (void)hipEventDestroy(ctx->copy_done);
    if (ctx->d_groups) (void)hipFree(ctx->d_groups);
    if (ctx->d_err) (void)hipFree(ctx->d_err);
    delete ctx;
}

int kvm_ctx_reserve(kvm_ctx* ctx, int64_t max_seqs, int64_t max_descs)
{
    if (!ctx || max_seqs < 0 || max_descs < 0) return KVM_EINVAL;
    if (max_seqs > kMaxSeqs || max_descs > kMaxDescs) return KVM_ERANGE;
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    const size_t per = std::max(sizeof(SeqRec), sizeof(MergeRec)) + sizeof(int64_t);
    int rc = stage_reserve(ctx, size_t(max_seqs + 64) * per);
    if (rc != KVM_OK) return rc;
    return grow_groups(ctx, (max_descs + kvm::kDescGroup - 1) / kvm::kDescGroup);
}

const char* kvm_ctx_last_error(const kvm_ctx* ctx) { return ctx ? ctx->last_error.c_str() : ""; }

int kvm_take_device_errors(kvm_ctx* ctx, int64_t* count)
{
    if (!ctx || !count) return KVM_EINVAL;
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail_hip(ctx, e, "hipDeviceSynchronize");
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
    SeqPlan plan;
    rc = plan_seqs(layout, num_layers, seqs, n, pack, &plan);
    if (rc != KVM_OK) return rc;
    if (plan.ntiles == 0) return KVM_OK;
    if (!pool) return KVM_EINVAL;
    const uint64_t bits = plan.align_bits | uint64_t(uintptr_t(pool)) | uint64_t(layout->row_bytes) |
                          uint64_t(layout->block_stride) | uint64_t(layout->side_stride) |
                          uint64_t(layout->layer_stride);
    const int unit = move_unit(bits);

    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* d = nullptr;
    int slot = 0;
    rc = stage_put(ctx, plan.bytes.data(), plan.bytes.size(), st, &d, &slot);
    if (rc != KVM_OK) return rc;
    const int64_t* tile0 = reinterpret_cast<const int64_t*>(d);
    const SeqRec* recs = reinterpret_cast<const SeqRec*>(d + plan.rec_offset);
    const PoolGeom g = geom_of(layout);
    hipError_t e;
    if (pack)
        e = kvm::launch_pack(unit, g, static_cast<const char*>(pool), num_layers, tile0, recs,
                             plan.nrec, plan.ntiles, ctx->d_err, st);
    else
        e = kvm::launch_unpack(unit, g, static_cast<char*>(const_cast<void*>(pool)), num_layers,
                               layer, tile0, recs, plan.nrec, plan.ntiles, ctx->d_err, st);
    if (e != hipSuccess) return fail_hip(ctx, e, pack ? "k_pack launch" : "k_unpack launch");
    return stage_mark(ctx, slot, st);
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
    const int32_t rows_per_tile = int32_t(std::max<int64_t>(1, kMergeTileBytes / row_bytes));
    std::vector<int64_t> tile0;
    std::vector<MergeRec> recs;
    int64_t tiles = 0;
    uint64_t bits = uint64_t(row_bytes);
    for (int32_t i = 0; i < n; ++i) {
        const kvm_merge_seq& m = seqs[i];
        if (m.t_hit < 0 || m.t_miss < 0 || m.hit_stride < 0 || m.miss_stride < 0 ||
            m.out_stride < 0)
            return KVM_EINVAL;
        if ((m.t_hit > 0 && !m.hit) || (m.t_miss > 0 && !m.miss)) return KVM_EINVAL;
        const int64_t t_all = m.t_hit + m.t_miss;
        if (t_all == 0) continue;
        if (!m.out) return KVM_EINVAL;
        tile0.push_back(tiles);
        tiles += (t_all + rows_per_tile - 1) / rows_per_tile;
        if (tiles > kMaxTiles) return KVM_ERANGE;
        MergeRec r;
        r.hit = static_cast<const char*>(m.hit);
        r.hit_stride = m.hit_stride;
        r.t_hit = m.t_hit;
        r.miss = static_cast<const char*>(m.miss);
        r.miss_stride = m.miss_stride;
        r.t_miss = m.t_miss;
        r.out = static_cast<char*>(m.out);
        r.out_stride = m.out_stride;
        recs.push_back(r);
        bits |= uint64_t(uintptr_t(m.out)) | uint64_t(m.out_stride);
        if (m.t_hit > 0) bits |= uint64_t(uintptr_t(m.hit)) | uint64_t(m.hit_stride);
        if (m.t_miss > 0) bits |= uint64_t(uintptr_t(m.miss)) | uint64_t(m.miss_stride);
    }
    if (tiles == 0) return KVM_OK;
    const int unit = move_unit(bits);
    const size_t padded = (tile0.size() + 63) / 64 * 64;
    const size_t rec_off = padded * sizeof(int64_t);
    std::vector<char> bytes(rec_off + recs.size() * sizeof(MergeRec), 0);
    std::memcpy(bytes.data(), tile0.data(), tile0.size() * sizeof(int64_t));
    std::memcpy(bytes.data() + rec_off, recs.data(), recs.size() * sizeof(MergeRec));

    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return KVM_EHIP;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* d = nullptr;
    int slot = 0;
    int rc = stage_put(ctx, bytes.data(), bytes.size(), st, &d, &slot);
    if (rc != KVM_OK) return rc;
    hipError_t e = kvm::launch_merge(unit, row_bytes, rows_per_tile,
                                     reinterpret_cast<const int64_t*>(d),
                                     reinterpret_cast<const MergeRec*>(d + rec_off),
                                     int32_t(recs.size()), tiles, st);
    if (e != hipSuccess) return fail_hip(ctx, e, "k_merge launch");
    return stage_mark(ctx, slot, st);
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
    const int64_t groups = (n_descs + kvm::kDescGroup - 1) / kvm::kDescGroup;
    int rc = grow_groups(ctx, groups);
    if (rc != KVM_OK) return rc;
    // Enough wavefronts to cover every CU several times over; each takes an
    // equal share of the bytes.
    const int32_t copy_blocks = ctx->num_cus * 8;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (ctx->copy_pending && ctx->copy_stream != st) {
        e = hipStreamWaitEvent(st, ctx->copy_done, 0);
        if (e != hipSuccess) return fail_hip(ctx, e, "hipStreamWaitEvent");
    }
    e = kvm::launch_batch_copy(
        static_cast<char*>(dst_base), dst_bytes, static_cast<const char*>(src_base), src_bytes,
        reinterpret_cast<const CopyDesc*>(descs), n_descs, ctx->d_groups,
        ctx->d_groups + ctx->group_cap, copy_blocks, ctx->d_err, st);
    if (e != hipSuccess) return fail_hip(ctx, e, "batch copy launch");
    e = hipEventRecord(ctx->copy_done, st);
    if (e != hipSuccess) return fail_hip(ctx, e, "hipEventRecord");
    ctx->copy_stream = st;
    ctx->copy_pending = true;
    return KVM_OK;
}

}  // extern "C"
