/*
 * pkv_oracle.h -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * fp64 host reference for paged-KV-cache store, decode attention and chunked
 * causal prefill attention.  Only tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  Layouts and citations: pkv_oracle.c.
 *
 * Every function returns PKO_OK (0) or a negative error code; on error
 * nothing has been written.
 */
#ifndef PKV_ORACLE_H
#define PKV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PKO_OK = 0,
    PKO_ERR_ARG = -1,       /* bad size, null pointer or head ratio */
    PKO_ERR_RANGE = -2,     /* slot, block id or context length out of range */
    PKO_ERR_DUPLICATE = -3, /* a slot repeats within one store call */
    PKO_ERR_ALLOC = -4      /* host allocation failed */
};

uint64_t pko_kv_bytes(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                      int64_t cached_tokens, int32_t bytes_per_element);

int pko_store(const uint16_t *k, const uint16_t *v, const int32_t *slot_mapping,
              int32_t num_tokens, uint16_t *k_cache, uint16_t *v_cache,
              int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
              int32_t block_size);

int pko_decode(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
               int32_t num_blocks, const int32_t *block_tables, int32_t max_blocks_per_seq,
               const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
               int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
               double *out, int nthreads);

int pko_prefill(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                int32_t num_blocks, const int32_t *block_tables, int32_t max_blocks_per_seq,
                const int32_t *cu_new_lens, const int32_t *context_lens, int32_t num_seqs,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size, float scale, double *out, int nthreads);

int pko_default_threads(void);

/* FP8 (OCP E4M3) cache with one fp32 scale per (token, KV head); see
 * pkv_oracle.c for the quantization rule. */
double pko_fp8_decode(uint8_t code);
uint8_t pko_fp8_encode(float y);
int pko_store_fp8(const uint16_t *k, const uint16_t *v, const int32_t *slot_mapping,
                  int32_t num_tokens, uint8_t *k_codes, uint8_t *v_codes, float *k_scales,
                  float *v_scales, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size);
/* Rotary position embedding of bf16 rows (see pkv_oracle.c for the formula). */
int pko_copy_blocks(uint8_t *const *pools, int32_t num_pools, int64_t block_bytes,
                    int32_t num_blocks, const int32_t *copies, int32_t num_pairs);
int pko_rope(const uint16_t *x, const int32_t *positions, int32_t num_rows, int32_t heads,
             int32_t head_dim, const float *cos_sin, int32_t max_positions, uint16_t *out);

int pko_decode_fp8(const uint16_t *q, const uint8_t *k_codes, const uint8_t *v_codes,
                   const float *k_scales, const float *v_scales, int32_t num_blocks,
                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                   const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                   double *out);
int pko_prefill_fp8(const uint16_t *q, const uint8_t *k_codes, const uint8_t *v_codes,
                    const float *k_scales, const float *v_scales, int32_t num_blocks,
                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                    const int32_t *cu_new_lens, const int32_t *context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, float scale, double *out, int nthreads);

#ifdef __cplusplus
}
#endif

#endif
