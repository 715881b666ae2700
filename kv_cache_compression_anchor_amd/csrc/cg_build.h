// Definitions of the table builder and the encoder (libcachegen): the per-lane
// quantiser, the statistics buffer, and their kernel launchers.
#pragma once

#include "cg_internal.h"

namespace cg {

// ----------------------------------------------------------------------------
// Per-lane quantiser (binary32, no contraction; identical in every kernel)
// ----------------------------------------------------------------------------
// The clamps are one v_med3_f32 each: for every value but NaN it equals
// min(max(r, lo), hi).  NaN arises only from non-finite input, which every
// caller flags and rejects; its code stays in range either way.
__device__ __forceinline__ int quant_anchor(float x, float inv_a) {
  float p = x * inv_a;
  float r = __builtin_rintf(p);
  r = __builtin_amdgcn_fmed3f(r, -127.0f, 127.0f);
  return (int)r;
}

// The delta's level rint(u) clamped to [-32, 31], u = (x - ahat) * inv_step,
// returned as the binary32 bits of u + 1.5 2^23 clamped to
// [kLevelBias - 32, kLevelBias + 31] (level = bits - kLevelBias): for
// |u| < 2^22 the sum is 1.5 2^23 + rint(u) exactly (its ulp is 1, and rounding
// to even agrees because 1.5 2^23 is even); beyond that the bits still order
// as u does (a negative sum has negative bits), so clamping the bits clamps
// the level.  One add and one v_med3_i32 instead of rint, a clamp and a
// conversion; callers fold the bias into their table or counter addresses.
constexpr int32_t kLevelBias = 0x4B400000;
__device__ __forceinline__ int32_t level_bits(float u) {
  return min(max(__builtin_bit_cast(int32_t, u + 12582912.0f), kLevelBias - 32), kLevelBias + 31);
}

// The anchor's code quant_anchor(x, inv_a) the same way: the bits of
// x inv_a + 1.5 2^23 clamped to kLevelBias -+ 127, equal to kLevelBias + the
// code for every finite x.  The low byte of the bits is the code's
// two's-complement byte (kLevelBias has a zero low byte), and anchor_of_bits
// gives the code as a binary32 exactly.
__device__ __forceinline__ int32_t anchor_bits(float x, float inv_a) {
  return min(max(__builtin_bit_cast(int32_t, x * inv_a + 12582912.0f), kLevelBias - 127),
             kLevelBias + 127);
}
__device__ __forceinline__ float anchor_of_bits(int32_t b) {
  return __builtin_bit_cast(float, b) - 12582912.0f;
}

struct StatsBuf {
  uint64_t* s1;    // sum of X = x*2^24 (two's complement)
  uint64_t* sa;    // sum over workgroups of (their sum of X^2) >> 40
  uint64_t* sc;    // sum over workgroups of (their sum of X^2) mod 2^40
  uint32_t* amax;  // max |x| as binary16 magnitude bits
  uint32_t* flags; // [0]: non-finite input, [1]: degenerate step, [2..3]: tables id,
                   // [4]: pooled count too large
};

hipError_t launch_stats(const uint16_t* x, int kv, int L, int T, int C, const StatsBuf& sb,
                        hipStream_t st);
hipError_t launch_finalize(const cg_params& p, const StatsBuf& sb, DevTables& t, hipStream_t st);
// acounts: [2][L][256] anchor-symbol counts, counted only when the tables code anchors
hipError_t launch_histogram(const uint16_t* x, int kv, const DevTables& t, uint32_t* counts,
                            uint32_t* acounts, hipStream_t st);
hipError_t launch_normalize(const DevTables& t, const uint32_t* counts, hipStream_t st);
// the anchor tables (no-op without coded anchors)
hipError_t launch_normalize_anchors(const DevTables& t, const uint32_t* acounts, hipStream_t st);
// pooled counts for a coarser table grouping (1 per layer, 2 per channel, 3 per
// (kv, quality)); pooled needs pooled_words() words; sets *overflow if a
// pooled count does not fit 32 bits
size_t pooled_words(const DevTables& t, int grouping);
hipError_t launch_pool(const DevTables& t, uint32_t* counts, int grouping, uint32_t* pooled,
                       uint32_t* overflow, hipStream_t st);
hipError_t launch_images(DevTables& t, hipStream_t st);
// digests the tables id needs: leaves, then middle digests
inline size_t id_leaves(size_t bytes) { return (bytes + kIdLeaf - 1) / kIdLeaf; }
inline size_t id_mids(size_t bytes) { return (id_leaves(bytes) + kIdFan - 1) / kIdFan; }
hipError_t launch_tables_id(const DevTables& t, uint64_t* scratch_digests, uint64_t* id_out,
                            hipStream_t st);

constexpr int kEncMaxBlobs = 16;  // blobs per encode launch (kernel-argument descriptors)
struct EncBlob {
  uint8_t* blob;      // output
  size_t cap;
  int32_t t0, tc, ng, q;
  BlobLayout lay;
  const uint16_t* img;       // cum images of quality q
  const float* inv_step;     // of quality q
  // per launch, for the launch's rows [row0, row0 + nrows) of the blob's payload rows:
  uint32_t* scratch;         // per 64-stream block: [swb / 4 units][64 lanes][4 words]
  uint32_t* lens;            // [nrows][C] words
  uint32_t* row_words;       // [nrows]
  uint32_t* block_words;     // [nrows][nblk] words of each 64-stream block
  // per blob, zero before its first launch: [0] payload words of the rows coded
  // so far, [1] too large for cap (sticky), [2] non-finite input
  uint32_t* status;
};
struct EncGroup {  // blobs of one quality coded by one workgroup (one wave each)
  int8_t blob[4];
};
struct EncodeArgs {
  const uint16_t* k;
  const uint16_t* v;
  int L, T, C, G, nblk, nblobs;
  int n_groups, waves;  // workgroups per (kv, layer, block) and their widest group
  int prio;             // 1: the launch's waves are all resident at once; level their progress
  // the payload rows this launch codes and packs: rows 0 .. 2L-1 are the delta
  // streams of (kv, layer) = (r / L, r % L) (k_encode), rows 2L .. 4L-1 the
  // anchor streams of coded-anchor blobs (k_anchor_encode).  A blob is coded by
  // launches over consecutive row ranges that do not straddle 2L, in order; the
  // one that ends at rows_total (2L, or 4L with coded anchors) also writes the
  // header and the padding
  int row0, nrows, rows_total;
  size_t swb;                // scratch words per stream of this launch's rows (a multiple of 4)
  const uint16_t* afreq;     // [2][L][256] anchor tables (coded anchors), else null
  const float* scale_a;
  const float* inv_a;
  uint64_t tables_id;
  EncGroup groups[kEncMaxBlobs];
  EncBlob b[kEncMaxBlobs];
  int ncu;     // compute units: workgroups ncu apart in launch order share one
  int lds_cu;  // LDS bytes of a compute unit
};
hipError_t launch_encode(const EncodeArgs& a, hipStream_t st);
// zeroes n words at p on st (a kernel, so that the clearing also works where
// a caller captures the stream into a graph)
hipError_t launch_zero_words(uint32_t* p, uint32_t n, hipStream_t st);

}  // namespace cg
