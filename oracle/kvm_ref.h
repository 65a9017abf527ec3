/*
 * kvm_ref.h -- oracle for the paged <-> Full Block KV-cache moves.
 *
 * TEST INFRASTRUCTURE. This is the plain, slow CPU definition that the HIP
 * library is checked against. Only the test suite, the smoke check and the
 * bench's CPU-baseline leg load it. It shares no code, header, table or
 * constant with the library, and the library never calls it.
 *
 * All payload is opaque bytes: nothing here reads a value as a number, so
 * bf16 NaN payloads, -0 and denormals pass through bit for bit.
 *
 * Return codes: 0 on success, -1 for a malformed argument, -2 for an index or
 * range outside its buffer, -5 for a precondition violation (duplicate block
 * ids, overlapping copy ranges). Nothing is written when a check fails.
 */
#ifndef KVM_REF_H
#define KVM_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Paged pool geometry. A token row of side s (K or V; one side for a single
 * latent), layer l, block n, row r starts at
 *   l*layer_stride + s*side_stride + n*block_stride + r*row_bytes
 * and is row_bytes long. layer_stride == 0 describes a one-layer slot pool
 * that every layer reuses. */
typedef struct {
    int32_t sides;
    int32_t block_tokens;
    int64_t row_bytes;
    int64_t block_stride;
    int64_t side_stride;
    int64_t layer_stride;
    int64_t num_blocks;
} kvm_ref_pool;

/* Full Block of one sequence: token-major [T][L][sides*row_bytes]; token t
 * starts at t*token_stride (token_stride 0 means the dense L*sides*row_bytes). */

int ref_pack_full(const uint8_t* pool, int64_t pool_bytes, const kvm_ref_pool* p,
                  int32_t num_layers, const int32_t* block_table, int64_t num_tokens,
                  uint8_t* full, int64_t full_bytes, int64_t token_stride);

int ref_unpack_layer(uint8_t* pool, int64_t pool_bytes, const kvm_ref_pool* p,
                     int32_t num_layers, int32_t layer, const int32_t* block_table,
                     int64_t num_tokens, const uint8_t* full, int64_t full_bytes,
                     int64_t token_stride);

/* Rows are row_bytes long; each buffer's size in bytes is given for bounds. */
int ref_merge_layer(int64_t row_bytes,
                    const uint8_t* hit, int64_t hit_bytes, int64_t hit_stride, int64_t t_hit,
                    const uint8_t* miss, int64_t miss_bytes, int64_t miss_stride, int64_t t_miss,
                    uint8_t* out, int64_t out_bytes, int64_t out_stride);

/* descs holds n triples (src_off, dst_off, nbytes). */
int ref_batch_copy(uint8_t* dst, uint64_t dst_bytes, const uint8_t* src, uint64_t src_bytes,
                   const uint64_t* descs, int64_t n);

/* Precondition check for a set of block tables used together: every entry in
 * [0, num_blocks) and no entry repeated across all tables. counts[i] entries
 * are read from tables + offsets[i]. */
int ref_check_block_tables(const int32_t* tables, const int64_t* offsets,
                           const int64_t* counts, int64_t n_tables, int64_t num_blocks);

/* Size bookkeeping. */
int64_t ref_blocks_for_tokens(int64_t tokens, int64_t block_tokens);
int64_t ref_objects_for_tokens(int64_t tokens, int64_t block_tokens, int64_t layers,
                               int64_t sides);
int64_t ref_kv_bytes(int64_t layers, int64_t tokens, int64_t heads, int64_t head_dim,
                     int64_t elem_bytes);

#ifdef __cplusplus
}
#endif

#endif /* KVM_REF_H */
