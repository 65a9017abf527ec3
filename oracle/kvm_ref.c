/*
 * kvm_ref.c -- oracle for the paged <-> Full Block KV-cache moves.
 *
 * TEST INFRASTRUCTURE. The plain CPU definition the HIP library is checked
 * against; only the test suite, the smoke check and the bench's CPU-baseline
 * leg use it. One memcpy per token row or per copy object, in the order the
 * definitions state them. No blocking, no threads, no shared code with the
 * library.
 *
 * What each function follows (page title, then section):
 *  - DualPath KV Loading, "Dual-Path Loading" key-objects table: the persisted
 *    Full Block is a [T_hit, L, C_KV] view; hit_layer[l] is its layer-l slice
 *    [T_hit, C_KV]; miss_layer[l] is [T_miss, C_KV]; complete_layer[l] is
 *    [T_all, C_KV], the hit rows followed by the miss rows.
 *  - DualPath KV Loading, "two read paths": the per-layer slice is written
 *    into an HBM layer slot; the hit and miss rows are concatenated by token.
 *  - DualPath KV Loading, design checklist and migration exercise: the Full
 *    Block <-> layer conversion keeps token, layer and KV-head order, and the
 *    result must agree byte for byte.
 *  - Tutti reading notes, prerequisites 3 (eq. 2): a paged block holds
 *    B_tokens tokens of [H, d]; a sequence's blocks are not contiguous and are
 *    found through its block table.
 *  - Tutti reading notes, prerequisites 5 (eq. 3-4): each block carries one K
 *    object and one V object per layer.
 *  - Tutti reading notes, prerequisites 2 (eq. 1): KV bytes = 2*L*T*H*d*e.
 *  - Tutti reading notes, design 1 (eq. 9) and Mooncake Ascend Transports,
 *    "why addresses need relocation": a copy is described by offsets into a
 *    known buffer plus a length, one entry per contiguous object.
 *
 * Readings where the pages leave the layout open: the pool is indexed
 * [layer][side][block][row] by strides; C_KV is the K heads followed by the
 * V heads (one side for a single latent); hit tokens are [0, T_hit) of the
 * sequence and miss tokens follow them.
 */
#include "kvm_ref.h"

#include <stdlib.h>
#include <string.h>

#define REF_OK 0
#define REF_EINVAL (-1)
#define REF_ERANGE (-2)
#define REF_EPRECOND (-5)

static int pool_ok(const kvm_ref_pool* p, int32_t num_layers)
{
    if (!p || num_layers <= 0) return 0;
    if (p->sides <= 0 || p->block_tokens <= 0 || p->row_bytes <= 0) return 0;
    if (p->block_stride < 0 || p->side_stride < 0 || p->layer_stride < 0) return 0;
    if (p->num_blocks <= 0) return 0;
    return 1;
}

/* Offset of token row r of (layer l, side s, block n) inside the pool. */
static int64_t pool_row_offset(const kvm_ref_pool* p, int64_t l, int64_t s, int64_t n, int64_t r)
{
    return l * p->layer_stride + s * p->side_stride + n * p->block_stride + r * p->row_bytes;
}

static int64_t dense_token_stride(const kvm_ref_pool* p, int32_t num_layers)
{
    return (int64_t)num_layers * p->sides * p->row_bytes;
}

/* Full Block row of (token t, layer l, side s): the token's L rows of C_KV
 * bytes follow each other, and side s of a layer row starts s*row_bytes in. */
static int64_t full_row_offset(const kvm_ref_pool* p, int64_t token_stride, int64_t t, int64_t l,
                               int64_t s)
{
    return t * token_stride + (l * p->sides + s) * p->row_bytes;
}

static int range_ok(int64_t off, int64_t len, int64_t size)
{
    return off >= 0 && len >= 0 && off <= size && len <= size - off;
}

/* Every slot and Full Block row the op will touch lies inside its buffer. */
static int check_rows(const kvm_ref_pool* p, int64_t pool_bytes, int32_t first_layer,
                      int32_t last_layer, const int32_t* bt, int64_t num_tokens,
                      int64_t full_bytes, int64_t token_stride)
{
    for (int64_t t = 0; t < num_tokens; ++t) {
        int32_t n = bt[t / p->block_tokens];
        if (n < 0 || n >= p->num_blocks) return 0;
        for (int32_t l = first_layer; l <= last_layer; ++l) {
            for (int32_t s = 0; s < p->sides; ++s) {
                int64_t po = pool_row_offset(p, l, s, n, t % p->block_tokens);
                int64_t fo = full_row_offset(p, token_stride, t, l, s);
                if (!range_ok(po, p->row_bytes, pool_bytes)) return 0;
                if (!range_ok(fo, p->row_bytes, full_bytes)) return 0;
            }
        }
    }
    return 1;
}

int ref_pack_full(const uint8_t* pool, int64_t pool_bytes, const kvm_ref_pool* p,
                  int32_t num_layers, const int32_t* block_table, int64_t num_tokens,
                  uint8_t* full, int64_t full_bytes, int64_t token_stride)
{
    if (!pool_ok(p, num_layers) || num_tokens < 0 || token_stride < 0) return REF_EINVAL;
    if (num_tokens == 0) return REF_OK;
    if (!pool || !full || !block_table) return REF_EINVAL;
    if (token_stride == 0) token_stride = dense_token_stride(p, num_layers);
    if (!check_rows(p, pool_bytes, 0, num_layers - 1, block_table, num_tokens, full_bytes,
                    token_stride))
        return REF_ERANGE;

    /* Full[t][l][s] <- pool[l][s][block_table[t / B]][t % B] for every token,
     * layer and side. */
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t block = block_table[t / p->block_tokens];
        int64_t row = t % p->block_tokens;
        for (int64_t l = 0; l < num_layers; ++l) {
            for (int64_t s = 0; s < p->sides; ++s) {
                memcpy(full + full_row_offset(p, token_stride, t, l, s),
                       pool + pool_row_offset(p, l, s, block, row), (size_t)p->row_bytes);
            }
        }
    }
    return REF_OK;
}

int ref_unpack_layer(uint8_t* pool, int64_t pool_bytes, const kvm_ref_pool* p,
                     int32_t num_layers, int32_t layer, const int32_t* block_table,
                     int64_t num_tokens, const uint8_t* full, int64_t full_bytes,
                     int64_t token_stride)
{
    if (!pool_ok(p, num_layers) || num_tokens < 0 || token_stride < 0) return REF_EINVAL;
    if (layer < 0 || layer >= num_layers) return REF_ERANGE;
    if (num_tokens == 0) return REF_OK;
    if (!pool || !full || !block_table) return REF_EINVAL;
    if (token_stride == 0) token_stride = dense_token_stride(p, num_layers);
    if (!check_rows(p, pool_bytes, layer, layer, block_table, num_tokens, full_bytes,
                    token_stride))
        return REF_ERANGE;

    /* pool[layer][s][block_table[t / B]][t % B] <- Full[t][layer][s] for the
     * first num_tokens tokens; every other slot keeps its bytes. */
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t block = block_table[t / p->block_tokens];
        int64_t row = t % p->block_tokens;
        for (int64_t s = 0; s < p->sides; ++s) {
            memcpy(pool + pool_row_offset(p, layer, s, block, row),
                   full + full_row_offset(p, token_stride, t, layer, s), (size_t)p->row_bytes);
        }
    }
    return REF_OK;
}

int ref_merge_layer(int64_t row_bytes,
                    const uint8_t* hit, int64_t hit_bytes, int64_t hit_stride, int64_t t_hit,
                    const uint8_t* miss, int64_t miss_bytes, int64_t miss_stride, int64_t t_miss,
                    uint8_t* out, int64_t out_bytes, int64_t out_stride)
{
    if (row_bytes <= 0 || t_hit < 0 || t_miss < 0) return REF_EINVAL;
    if (hit_stride < 0 || miss_stride < 0 || out_stride < 0) return REF_EINVAL;
    if ((t_hit > 0 && !hit) || (t_miss > 0 && !miss) || (t_hit + t_miss > 0 && !out))
        return REF_EINVAL;
    for (int64_t t = 0; t < t_hit; ++t) {
        if (!range_ok(t * hit_stride, row_bytes, hit_bytes)) return REF_ERANGE;
        if (!range_ok(t * out_stride, row_bytes, out_bytes)) return REF_ERANGE;
    }
    for (int64_t i = 0; i < t_miss; ++i) {
        if (!range_ok(i * miss_stride, row_bytes, miss_bytes)) return REF_ERANGE;
        if (!range_ok((t_hit + i) * out_stride, row_bytes, out_bytes)) return REF_ERANGE;
    }

    /* complete = hit rows 0..T_hit-1, then miss rows as rows T_hit..T_all-1. */
    for (int64_t t = 0; t < t_hit; ++t)
        memcpy(out + t * out_stride, hit + t * hit_stride, (size_t)row_bytes);
    for (int64_t i = 0; i < t_miss; ++i)
        memcpy(out + (t_hit + i) * out_stride, miss + i * miss_stride, (size_t)row_bytes);
    return REF_OK;
}

typedef struct {
    uint64_t begin;
    uint64_t end;
} ref_span;

static int span_cmp(const void* a, const void* b)
{
    const ref_span* x = (const ref_span*)a;
    const ref_span* y = (const ref_span*)b;
    if (x->begin != y->begin) return x->begin < y->begin ? -1 : 1;
    if (x->end != y->end) return x->end < y->end ? -1 : 1;
    return 0;
}

/* Sorted, pairwise-disjoint spans: does any of them meet [b, e)? */
static int meets_any(const ref_span* sorted, int64_t m, uint64_t b, uint64_t e)
{
    /* first span whose end lies beyond b */
    int64_t lo = 0, hi = m;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (sorted[mid].end <= b) lo = mid + 1;
        else hi = mid;
    }
    return lo < m && sorted[lo].begin < e;
}

int ref_batch_copy(uint8_t* dst, uint64_t dst_bytes, const uint8_t* src, uint64_t src_bytes,
                   const uint64_t* descs, int64_t n)
{
    if (n < 0) return REF_EINVAL;
    if (n == 0) return REF_OK;
    if (!descs || !dst || !src) return REF_EINVAL;

    /* Every object lies inside its buffer. */
    for (int64_t k = 0; k < n; ++k) {
        uint64_t so = descs[3 * k], d_o = descs[3 * k + 1], len = descs[3 * k + 2];
        if (so > src_bytes || len > src_bytes - so) return REF_ERANGE;
        if (d_o > dst_bytes || len > dst_bytes - d_o) return REF_ERANGE;
    }

    /* Destinations are pairwise disjoint, and when source and destination are
     * one buffer no destination meets a source; then the order of the copies
     * does not matter and the result is unique. */
    ref_span* spans = (ref_span*)malloc(sizeof(ref_span) * (size_t)n);
    if (!spans) return REF_EINVAL;
    int64_t m = 0;
    for (int64_t k = 0; k < n; ++k) {
        uint64_t len = descs[3 * k + 2];
        if (len == 0) continue;
        spans[m].begin = descs[3 * k + 1];
        spans[m].end = descs[3 * k + 1] + len;
        ++m;
    }
    qsort(spans, (size_t)m, sizeof(ref_span), span_cmp);
    int bad = 0;
    for (int64_t i = 1; i < m && !bad; ++i)
        if (spans[i].begin < spans[i - 1].end) bad = 1;
    if (!bad && (const uint8_t*)dst == src) {
        for (int64_t k = 0; k < n && !bad; ++k) {
            uint64_t len = descs[3 * k + 2];
            if (len && meets_any(spans, m, descs[3 * k], descs[3 * k] + len)) bad = 1;
        }
    }
    free(spans);
    if (bad) return REF_EPRECOND;

    for (int64_t k = 0; k < n; ++k) {
        uint64_t so = descs[3 * k], d_o = descs[3 * k + 1], len = descs[3 * k + 2];
        if (len) memcpy(dst + d_o, src + so, (size_t)len);
    }
    return REF_OK;
}

static int id_cmp(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

int ref_check_block_tables(const int32_t* tables, const int64_t* offsets, const int64_t* counts,
                           int64_t n_tables, int64_t num_blocks)
{
    if (n_tables < 0 || num_blocks <= 0) return REF_EINVAL;
    int64_t total = 0;
    for (int64_t i = 0; i < n_tables; ++i) {
        if (counts[i] < 0 || offsets[i] < 0) return REF_EINVAL;
        total += counts[i];
    }
    if (total == 0) return REF_OK;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)total);
    if (!ids) return REF_EINVAL;
    int64_t m = 0;
    for (int64_t i = 0; i < n_tables; ++i)
        for (int64_t j = 0; j < counts[i]; ++j) ids[m++] = tables[offsets[i] + j];
    int rc = REF_OK;
    for (int64_t k = 0; k < m; ++k)
        if (ids[k] < 0 || ids[k] >= num_blocks) rc = REF_ERANGE;
    if (rc == REF_OK) {
        qsort(ids, (size_t)m, sizeof(int32_t), id_cmp);
        for (int64_t k = 1; k < m; ++k)
            if (ids[k] == ids[k - 1]) rc = REF_EPRECOND;
    }
    free(ids);
    return rc;
}

int64_t ref_blocks_for_tokens(int64_t tokens, int64_t block_tokens)
{
    if (tokens <= 0 || block_tokens <= 0) return 0;
    return (tokens + block_tokens - 1) / block_tokens;
}

int64_t ref_objects_for_tokens(int64_t tokens, int64_t block_tokens, int64_t layers, int64_t sides)
{
    /* one object per (layer, side) per block */
    return sides * layers * ref_blocks_for_tokens(tokens, block_tokens);
}

int64_t ref_kv_bytes(int64_t layers, int64_t tokens, int64_t heads, int64_t head_dim,
                     int64_t elem_bytes)
{
    /* K and V, for every layer, token, head and head-dim element */
    return 2 * layers * tokens * heads * head_dim * elem_bytes;
}
