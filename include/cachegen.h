/*
 * cachegen.h — C ABI of the MI355X (gfx950) KV-cache codec library libcachegen.so.
 *
 * The codec follows CacheGen (arXiv 2310.07240):
 *   - the encoder turns a KV cache into a compact bitstream (gptget abstract;
 *     CacheGen blog, section 2.1 pseudocode: a function from a KV tensor to a
 *     bitstream);
 *   - tokens are coded as deltas against an 8-bit anchor token, one anchor per
 *     group of ten (CacheGen blog, section 2.1 pseudocode; sciencestack TL;DR on
 *     the locality of neighbouring tokens);
 *   - the delta step depends on the layer group, 0.5 / 1.0 / 1.5 channel stds for
 *     shallow / medium / deep layers (CacheGen blog, sections 1 and 2.1;
 *     sciencestack TL;DR on quantisation that depends on the layer);
 *   - the symbols are arithmetic-coded with probability tables kept per
 *     (layer, channel) (CacheGen blog, section 1; sciencestack Figure 5);
 *   - the context is cut into 1.5K-token chunks, each pre-encoded at quality
 *     H, M or L, and decoded on the GPU, pipelined with its transfer
 *     (CacheGen blog, section 2.2; gptget 方法详解).
 *
 * Tensors: K and V are each [layers][tokens][channels] IEEE binary16, contiguous,
 * channels fastest, in device memory.
 *
 * Memory ownership: every pointer argument is owned by the caller, except the
 * cg_tables handle, which the library allocates (device copies of the tables,
 * from a stream-ordered memory pool it keeps per device, which holds on to the
 * blocks it has cached until the process ends) and cg_tables_free releases
 * (after waiting for the device).  Building tables and encoding each use one
 * workspace per device (statistics, symbol counts, digests; the encoder's
 * stream scratch, lengths and status words), grown to the largest build or
 * batch and kept until the process ends; builds on one device take turns on
 * theirs, and so do encode batches.  Device buffers passed to an *_async /
 * streamed call must stay valid until the stream has executed the work.
 *
 * Streams: a `void* stream` is a hipStream_t (NULL = the legacy default stream).
 * A handle is used on the device that built or deserialized it; the library
 * switches to that device for the call and restores the caller's device.
 *
 * Errors: every int-returning call returns CG_OK (0) or a negative CG_E_* code
 * and never aborts; cg_last_error() gives the message of the calling thread's
 * last failure.  Arguments are validated before any GPU work is enqueued.
 */
#ifndef CACHEGEN_H
#define CACHEGEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CG_OK = 0,
  CG_E_INVAL = -1,    /* bad argument, shape or parameter; non-finite input */
  CG_E_NOMEM = -2,    /* device or host allocation failed */
  CG_E_HIP = -3,      /* HIP runtime error (message in cg_last_error) */
  CG_E_CORRUPT = -4,  /* a blob failed validation while decoding */
  CG_E_CAPACITY = -5, /* output buffer too small */
  CG_E_MISMATCH = -6  /* blob made for other tables, or quality not in the tables */
};

enum { CG_Q_H = 0, CG_Q_M = 1, CG_Q_L = 2 }; /* quality levels (CacheGen blog 2.2) */

/* Codec parameters.  Groups restart at every chunk; the first token of a group
 * is its anchor.  Layer l uses layer_step[g] where g is the first group with
 * l < layer_group_end[g]; quality q multiplies the step by quality_mult[q]. */
typedef struct {
  int32_t layers, tokens, channels; /* each of K and V is [layers][tokens][channels] */
  int32_t chunk_tokens;             /* 1 .. 65536 (1536 in the pages' setting); one chunk of
                                       one layer, min(chunk_tokens, tokens) x channels x 2
                                       bytes, must be below 4 GiB */
  int32_t group_tokens;             /* 1 .. chunk_tokens (10 in the pages' setting) */
  int32_t n_layer_groups;           /* 1 .. 3, or 0 for the default: three groups with ends
                                       floor(10 L / 32), floor(20 L / 32), L (the pages'
                                       layers 1-10 / 11-20 / 21-32 scaled to L >= 4 layers),
                                       layer_step[0..2] their steps; layer_group_end is then
                                       ignored and cg_tables_params reports the ends used */
  int32_t layer_group_end[3];       /* exclusive ends, increasing, last == layers */
  float layer_step[3];              /* delta step per layer group, channel-std units */
  float quality_mult[3];            /* step multiplier of H, M, L */
  uint32_t quality_mask;            /* bit q set: build tables for quality q */
  int32_t anchor_coding;            /* 0: anchors stored as raw bytes (tables version 1,
                                       blobs version 2); 1: anchors range-coded with one
                                       256-symbol table per (kv, layer) counted like the
                                       delta tables (tables version 2, blobs version 3;
                                       channels x tokens must stay below 2^32) */
} cg_params;

/* Header fields of one chunk blob, read from host memory by cg_chunk_info_parse. */
typedef struct {
  int32_t layers, channels, total_tokens;
  int32_t token_offset;  /* first token of the chunk in the [tokens] axis */
  int32_t chunk_tokens;  /* tokens in this chunk (the last chunk may be short) */
  int32_t group_tokens, n_groups, quality;
  uint32_t payload_words;
  uint32_t version;      /* blob format: 2 raw anchors, 3 range-coded anchors */
  uint64_t tables_id;    /* identity of the tables the blob was coded with */
  uint64_t blob_bytes;   /* total size of the blob */
} cg_chunk_info;

typedef struct cg_tables cg_tables; /* opaque, library-owned */

/* Builds the per-(kv, layer, channel) tables from the K/V pair they will code:
 * channel statistics (exact integer moments), anchor scales, delta steps, and,
 * for each quality in quality_mask, the frequency table of the delta symbols
 * over every chunk (CacheGen blog, section 1: symbol probabilities counted per
 * layer-channel combination).  k_dev, v_dev: device fp16 [layers][tokens][channels].
 * Runs on `stream`, then waits for it.  Non-finite input gives CG_E_INVAL.
 * On success *out receives a new handle. */
int cg_build_tables(const cg_params* params, const void* k_dev, const void* v_dev,
                    void* stream, cg_tables** out);

/* Table groupings: which (kv, quality, layer, channel) tables share pooled
 * symbol statistics.  CG_GROUP_LAYER_CHANNEL (one table per layer and channel,
 * the pages' choice: CacheGen blog, section 1) is what cg_build_tables builds;
 * the coarser ones exist to measure what that choice is worth. */
enum {
  CG_GROUP_LAYER_CHANNEL = 0, /* per (kv, quality, layer, channel) */
  CG_GROUP_LAYER = 1,         /* counts pooled over the channels of a layer */
  CG_GROUP_CHANNEL = 2,       /* counts pooled over the layers of a channel */
  CG_GROUP_GLOBAL = 3         /* counts pooled over all layers and channels */
};

/* cg_build_tables with the delta-symbol counts pooled over a coarser group
 * before they are turned into frequency tables: every table of a group is then
 * the group's table (scales and steps stay per layer and channel, and the
 * tables keep their layout, so encoding and decoding are unchanged).
 * CG_E_INVAL also for an unknown grouping and for a pooled count of one symbol
 * that does not fit 32 bits. */
int cg_build_tables_grouped(const cg_params* params, int32_t grouping, const void* k_dev,
                            const void* v_dev, void* stream, cg_tables** out);

/* Releases a handle and its device memory (NULL is allowed).  The caller makes
 * sure no enqueued work still uses it. */
void cg_tables_free(cg_tables* tables);

/* Serialized tables (the codebook shipped to a decoder): CGT1 version 1, or
 * version 2 with the anchor tables of coded anchors.  cg_tables_serialize
 * copies them into the host buffer `buf` of `cap` bytes; *len receives the size
 * (call with buf == NULL to query it).  cg_tables_deserialize validates host
 * bytes (header, parameters, size, every scale, step and frequency table) and
 * uploads them to the current device; CG_E_INVAL for anything malformed. */
int cg_tables_serialize(const cg_tables* tables, void* buf, size_t cap, size_t* len);
int cg_tables_deserialize(const void* buf, size_t len, cg_tables** out);

/* The tables' identity (stamped into blobs) and their parameters. */
uint64_t cg_tables_id(const cg_tables* tables);
int cg_tables_params(const cg_tables* tables, cg_params* out);

/* Number of chunks, and the worst-case size of chunk `chunk`'s blob. */
int cg_num_chunks(const cg_tables* tables, int32_t* n_chunks);
int cg_encode_bound(const cg_tables* tables, int32_t chunk, size_t* max_bytes);

/* Encodes chunk `chunk` of the K/V pair at `quality` into one blob written at
 * the device address out_dev (`cap` bytes; the blob needs at most
 * cg_encode_bound bytes, CG_E_CAPACITY if it does not fit).  The tensors must be
 * the ones the tables were built from (same shape).  One stream per
 * (kv, layer, channel): the group's first token as an int8 anchor, the others
 * as range-coded delta symbols (CacheGen blog, section 2.1 stages 1-3).
 * Runs on `stream` and waits for it; *out_len receives the blob size.
 * Encodes on one device take turns on its encode workspace. */
int cg_encode(const cg_tables* tables, const void* k_dev, const void* v_dev,
              int32_t chunk, int32_t quality, void* out_dev, size_t cap,
              size_t* out_len, void* stream);

/* Encodes n (chunk, quality) blobs of the same K/V as cg_encode does, in as few
 * kernel launches as the encode scratch allows (all streams of up to 16 blobs in
 * flight together), waiting for the stream once at the end.  outs_dev[i] (caps[i]
 * bytes) receives blob i and out_lens[i] its size (0 for a blob that failed).
 * Every argument is checked before any launch; on a per-blob failure (capacity,
 * non-finite input) the first such error is returned after the others finished. */
int cg_encode_batch(const cg_tables* tables, const void* k_dev, const void* v_dev, int32_t n,
                    const int32_t* chunks, const int32_t* qualities, void* const* outs_dev,
                    const size_t* caps, size_t* out_lens, void* stream);

/* For callers that cannot allocate device memory (harnesses that forbid
 * hipMalloc, serving loops that must not allocate): cg_encode_batch with the
 * same arguments, results and errors, that allocates nothing.  Its encode
 * scratch is a 256 MiB array of static device memory, one per GPU, held from
 * the library's load until the process ends; a blob is coded over as many
 * (kv, layer) rows at a time as fit in it, one blob after another.  A chunk
 * whose single (kv, layer) row needs more scratch than that (about
 * channels x 64 x chunk_tokens x 15 / 32 words) fails with CG_E_CAPACITY
 * before any launch.  Calls on one GPU share the array: the library lets one
 * call at a time use it and holds it until the call's stream has finished, so
 * calls that would overlap on one GPU take turns.  Waits for the stream after
 * every blob. */
int cg_encode_batch_noalloc(const cg_tables* tables, const void* k_dev, const void* v_dev,
                            int32_t n, const int32_t* chunks, const int32_t* qualities,
                            void* const* outs_dev, const size_t* caps, size_t* out_lens,
                            void* stream);

/* Parses and checks a blob header from host memory (len >= 64). Host only.
 * CG_E_INVAL for a header that is not CGK1 version 2 (raw anchors) or 3
 * (range-coded anchors), whose fields disagree with each other, whose blob
 * would exceed 4 GiB, or whose chunk of one layer (chunk_tokens x channels x 2
 * bytes) is 4 GiB or more.  out->version is the blob's format version. */
int cg_chunk_info_parse(const void* blob_host, size_t len, cg_chunk_info* out);

/* Decodes n blobs (device addresses blobs_dev[i]) into K/V fp16
 * [layers][total_tokens][channels] at k_out_dev / v_out_dev; each blob writes its
 * own token range.  The blobs' headers are read back to the host first.  Runs on
 * `stream`, waits for it, and returns CG_E_CORRUPT if a blob failed validation
 * on the device. */
int cg_decode(const cg_tables* tables, int32_t n, const void* const* blobs_dev,
              const size_t* lens, void* k_out_dev, void* v_out_dev, void* stream);

/* Enqueue-only decode (gptget 方法详解: GPU decoding of the received bitstream).
 * infos[i] is the parsed header of blobs_dev[i] (cg_chunk_info_parse on a host
 * copy); the device blob must hold the same bytes.  Bit 0 of *status_dev
 * (caller-owned device uint32, never cleared by the library) is set if a
 * stream of a blob is inconsistent (offsets past the payload, impossible code
 * value).  Corrupt payloads never cause out-of-bounds accesses.  A blob whose
 * format (cg_chunk_info.version) differs from the tables' anchor coding is
 * CG_E_MISMATCH.  With coded anchors the call first decodes the anchor
 * streams into 2 x layers x n_groups x channels bytes per blob, allocated
 * stream-ordered on `stream` from a memory pool the library keeps per device
 * (hipMallocFromPoolAsync) and freed there after the decode (hipFreeAsync);
 * the pool keeps the blocks it has held until the process ends.  The other
 * decode entry points do the same. */
int cg_decode_async(const cg_tables* tables, int32_t n, const void* const* blobs_dev,
                    const cg_chunk_info* infos, void* k_out_dev, void* v_out_dev,
                    uint32_t* status_dev, void* stream);

/* Enqueue-only decode straight into paged K/V pools (gptget 方法详解: the
 * receiver's GPU decoder hands the cache to the model; a serving engine keeps
 * that cache in fixed-size pages).  The pools k_pool_dev / v_pool_dev are fp16
 * [layers][num_pages][page_tokens][channels] (each layer's pages contiguous),
 * caller-owned.  Context token t is written to row t % page_tokens of page
 * block_table_dev[t / page_tokens]; block_table_dev is a caller-owned device
 * int32 array of n_blocks entries, read while the decode runs, which must name
 * distinct pages for the blocks the blobs cover (rows of two blocks that share
 * a page overwrite each other).  Rows and pages no blob writes keep their
 * contents.  An entry outside [0, num_pages) is not written: its rows are
 * skipped and bit 1 of *status_dev is set; bit 0 is set as in cg_decode_async.
 * The decoded values equal cg_decode_async's bit for bit.
 * CG_E_INVAL: NULL argument; page_tokens not a power of two in [1, 65536];
 * num_pages or n_blocks < 1; a layer's pool of 2 GiB or more; a block table
 * shorter than ceil((token_offset + chunk_tokens) / page_tokens) for some blob;
 * group_tokens > 64, or a last 64-channel block with fewer than group_tokens
 * channels (channels % 64 in [1, group_tokens)).  Header mismatches as in
 * cg_decode_async. */
int cg_decode_paged_async(const cg_tables* tables, int32_t n, const void* const* blobs_dev,
                          const cg_chunk_info* infos, void* k_pool_dev, void* v_pool_dev,
                          int64_t num_pages, int32_t page_tokens, const int32_t* block_table_dev,
                          int64_t n_blocks, uint32_t* status_dev, void* stream);

/* Chunk pipeline (gptget 方法详解: decoding pipelined with the transfer; CacheGen
 * blog 2.2: chunk-by-chunk streaming).  blobs_host[i] are host blobs (pinned
 * memory gives asynchronous copies); each is copied into a slot of the device
 * staging buffer (staging_cap bytes; at least two blobs' worth overlaps copy and
 * decode) on copy_stream and decoded on compute_stream once its copy has
 * landed; a slot is reused only after its previous decode finished.  Enqueue
 * only; the work is complete when compute_stream is. */
int cg_decode_streamed(const cg_tables* tables, int32_t n, const void* const* blobs_host,
                       const cg_chunk_info* infos, void* k_out_dev, void* v_out_dev,
                       void* staging_dev, size_t staging_cap, uint32_t* status_dev,
                       void* copy_stream, void* compute_stream);

/* Bandwidth-adaptive choice of the next chunk's version (CacheGen blog 2.2,
 * the bandwidth-adaptive selection formula: each chunk's version is chosen
 * from the measured bandwidth B and the service-level objective).  For every
 * version q that exists (bytes_left[q] > 0) the ratio
 *     r[q] = (budget_ms - decode_ms_left[q]) / (bytes_left[q] / bandwidth_bpms)
 * is the SLO time left after decoding over the time to send the rest of the
 * context at q.  The choice is the highest quality (H, then M, then L) with
 * r[q] >= 1, i.e. whose transfer fits what is left of the SLO; when none fits,
 * the version that is done soonest, the smallest bytes_left[q] / bandwidth_bpms
 * + decode_ms_left[q] (the first in H, M, L order on a tie).
 *   budget_ms        SLO minus the time this context has already taken (may be
 *                    negative: then nothing fits)
 *   bandwidth_bpms   bytes per millisecond, > 0 and finite (the throughput the
 *                    previous chunk saw, or a prior for the first chunk)
 *   bytes_left[q]    bytes of this chunk and all later ones at version q (H, M,
 *                    L); 0 marks a version that was not encoded
 *   decode_ms_left[q] their decode time, >= 0
 * Host only; ratios are computed in binary64 in exactly this order.  Writes the
 * chosen quality (CG_Q_H / CG_Q_M / CG_Q_L) to *quality_out and, when ratio_out
 * is not NULL, r[q] for each version (0 for a missing one) to ratio_out[0..2].
 * CG_E_INVAL: NULL in or quality_out, a NaN budget, a bandwidth that is not
 * positive and finite, a negative or non-finite decode time, or no version. */
typedef struct {
  double budget_ms;
  double bandwidth_bpms;
  uint64_t bytes_left[3];
  double decode_ms_left[3];
} cg_chunk_plan_in;
int cg_plan_chunk(const cg_chunk_plan_in* in, int32_t* quality_out, double* ratio_out);

/* For long-running processes: frees the device memory the library keeps
 * between calls, on every device it has used — the table-build and encode
 * workspaces (and their pinned host words), and the blocks its per-device
 * memory pool has cached that no tables handle or enqueued decode holds (the
 * blocks in use stay).  Waits for each such device to finish its work first;
 * calls on other threads that need a workspace wait for it, and the next call
 * that needs one allocates it again.  The static scratch of
 * cg_encode_batch_noalloc is not released (it lives until the process ends).
 * CG_OK, or CG_E_HIP if a device could not be selected, synchronised or its
 * pool trimmed (the other devices are still released). */
int cg_release_cached(void);

/* Message of the calling thread's last error ("" if none). */
const char* cg_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CACHEGEN_H */
