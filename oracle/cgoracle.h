/*
 * CPU oracle of the CacheGen KV-cache tensor codec — TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the package smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header, table or constant generator
 * with the GPU library: it is written from the method's description alone.
 *
 * Method (CacheGen: KV Cache Compression and Streaming, arXiv 2310.07240):
 *   - token-wise locality: code each token as a delta against an anchor token
 *     (sciencestack TL;DR; CacheGen blog, section 1 and the section 2.1 pseudocode,
 *     whose anchor is the first token of a group of ten, quantized to 8 bits);
 *   - layer-wise sensitivity: the delta step grows with layer depth, 0.5 / 1.0 /
 *     1.5 for shallow / medium / deep layers (CacheGen blog, sections 1 and 2.1);
 *   - arithmetic coding with symbol statistics kept per (layer, channel)
 *     (CacheGen blog, section 1 "grouped arithmetic coding"; sciencestack
 *     TL;DR and Figure 5);
 *   - 1.5K-token chunks, each pre-encoded at three qualities H/M/L
 *     (CacheGen blog, section 2.2).
 * Every step the pages leave open is fixed by the readings listed in the
 * repository's design notes; each function below names the one it follows.
 */
#ifndef CGORACLE_H
#define CGORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t layers, tokens, channels;
  int32_t chunk_tokens, group_tokens;
  int32_t n_layer_groups;
  int32_t layer_group_end[3];
  float layer_step[3];
  float quality_mult[3];
  uint32_t quality_mask;
  /* 1: anchors range-coded with one 256-symbol table per (kv, layer) (tables
   * version 2, blob version 3); 0: anchors stored as raw bytes */
  int32_t anchor_coding;
} cgo_params;

/* IEEE 754 binary16 conversions */
float cgo_f16_to_f32(uint16_t h);
uint16_t cgo_f32_to_f16(float f);
void cgo_f16_to_f32_array(const uint16_t* in, float* out, int64_t n);
void cgo_f32_to_f16_array(const float* in, uint16_t* out, int64_t n);
/* reconstruction of delta tokens: the binary16 nearest to the exact
 * ahat + (s - 32) * step, ties to even */
void cgo_dequant_delta_array(const uint8_t* s, const float* step, const float* ahat,
                             uint16_t* out, int64_t n);

/* generic range coder, P = 15, alphabet of nsym <= 256 symbols */
size_t cgo_rc_bound(int64_t n);
int cgo_rc_encode(const uint8_t* sym, int64_t n, const uint16_t* freq, int nsym,
                  uint8_t* out, size_t cap, size_t* out_len);
int cgo_rc_decode(const uint8_t* buf, size_t buflen, int64_t n, const uint16_t* freq,
                  int nsym, uint8_t* sym, size_t* consumed, int* corrupt);
void cgo_normalize(const uint32_t* counts, int nsym, uint16_t* freq);
void cgo_normalize_tables(const uint32_t* counts, int64_t ntab, uint16_t* freq);

/* per (l, c) statistics of one [L][T][C] fp16 tensor */
void cgo_channel_stats(const uint16_t* x, int L, int T, int C, double* sigma,
                       float* absmax, int* nonfinite);

/* tables */
size_t cgo_tables_size(const cgo_params* p);
int cgo_build_tables(const cgo_params* p, const uint16_t* k, const uint16_t* v,
                     int nthreads, uint8_t* out, size_t cap, size_t* len,
                     uint32_t* counts_out);
uint64_t cgo_fnv1a64(const uint8_t* data, size_t n);
uint64_t cgo_tables_id(const uint8_t* data, size_t n);

/* chunks */
int cgo_chunk_geometry(const uint8_t* tables, size_t tlen, int chunk, int32_t* t0,
                       int32_t* tc, int32_t* n_groups);
size_t cgo_encode_bound(const uint8_t* tables, size_t tlen, int chunk);
int cgo_encode_chunk(const uint8_t* tables, size_t tlen, const uint16_t* k,
                     const uint16_t* v, int chunk, int q, int nthreads, uint8_t* out,
                     size_t cap, size_t* len);
int cgo_chunk_symbols(const uint8_t* tables, size_t tlen, const uint16_t* k,
                      const uint16_t* v, int chunk, int q, int8_t* anchors,
                      uint8_t* syms);
int cgo_decode_blob(const uint8_t* tables, size_t tlen, const uint8_t* blob, size_t blen,
                    uint16_t* k_out, uint16_t* v_out, int nthreads, int* corrupt);
int cgo_decode_blob_symbols(const uint8_t* tables, size_t tlen, const uint8_t* blob,
                            size_t blen, uint8_t* syms, int* corrupt);

/* one stream (kv, l, c) of one chunk, for sampled checks at full size */
int cgo_stream_encode(const uint8_t* tables, size_t tlen, int kv, int l, int c, int q,
                      const uint16_t* x, int tc, int8_t* anchors, uint8_t* out,
                      size_t cap, size_t* len);
int cgo_stream_decode(const uint8_t* tables, size_t tlen, int kv, int l, int c, int q,
                      const int8_t* anchors, int tc, const uint8_t* bytes,
                      size_t nbytes, uint16_t* y, int* corrupt);

#ifdef __cplusplus
}
#endif
#endif
