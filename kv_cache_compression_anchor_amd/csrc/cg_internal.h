// Internal definitions of libcachegen shared by every device part: conversions,
// the decoder's launcher (container layouts and format constants are in
// cg_format.h).  The table builder's and encoder's own definitions are in
// cg_build.h.  Device code targets gfx950
// (wave64, 160 KB LDS per CU).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cachegen.h"
#include "cg_format.h"

namespace cg {

constexpr uint32_t kBufRsrcWord3 = 0x00020000u;  // raw buffer, gfx9 family

// the anchor's reconstruction, shared by the encoder's closed loop and the decoder
__device__ __forceinline__ float anchor_value(int a, float scale_a) { return (float)a * scale_a; }

// binary16 <-> binary32 with the hardware conversions (round to nearest even,
// binary16 subnormals kept)
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// The operand is made opaque first: otherwise the compiler may fold the
// conversion into the FMA that produced it (v_fma_mixlo_f16), which rounds the
// exact sum once to binary16 instead of rounding to binary32 first.
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  asm volatile("" : "+v"(f));
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// 24x24-bit unsigned multiply (v_mul_u32_u24).  HIP's __umul24 is declared to
// return int, which would sign-extend products >= 2^31 when widened.
__device__ __forceinline__ uint32_t mul24(uint32_t a, uint32_t b) {
  return static_cast<uint32_t>(__umul24(a, b));
}

// LDS slot of a lane inside a 64-wide table row: lanes l and l+32 share one
// 4-byte bank word, so a 16-bit gather by 32 lanes touches 32 distinct banks.
__host__ __device__ __forceinline__ int lane_slot(int lane) { return 2 * (lane & 31) + (lane >> 5); }

// ----------------------------------------------------------------------------
// Kernel launchers (defined in the .hip files)
// ----------------------------------------------------------------------------
struct DevTables {
  int L = 0, T = 0, C = 0, CH = 0, G = 0, nblk = 0;
  uint32_t mask = 0;
  TabLayout lay;
  uint8_t* ser = nullptr;                       // serialized tables, device copy
  uint16_t* img[3] = {nullptr, nullptr, nullptr};  // cum images [2][L][nblk][65][64]
};

constexpr int kDecMaxChunks = 24;
struct DecChunk {
  const uint8_t* blob;
  uint32_t blob_bytes;
  int32_t t0, tc, ng, q;
  uint32_t off_len, off_pay, W;
  // the chunk's anchors, i8 [2][L][ng][C]: the blob's raw anchor section, or
  // with coded anchors where k_anchor_decode wrote them
  const int8_t* anc;
  uint32_t anc_bytes;
};
struct DecGroup {  // chunks of one quality decoded by one workgroup (one wave each)
  int8_t chunk[4];
};
struct DecodeArgs {
  int L, T, C, G, nblk, waves, n_groups;
  DecGroup groups[kDecMaxChunks];
  DecChunk chunks[kDecMaxChunks];
  const uint16_t* img[3];
  const float* scale_a;
  const float* step[3];
  uint16_t* k_out;  // [L][T][C], or when paged the pools [L][num_pages][page][C]
  uint16_t* v_out;
  uint32_t* status;
  // 1: the workgroups have one more wave, which only reads the streams of its
  // block ahead of the decoding waves (to warm the caches); 0: no such wave
  int warm_wave;
  // always zero: the warming wave ANDs the values it read with it, so that its
  // loads are kept without their values deciding anything
  uint32_t sink_mask;
  // paged output: context token t goes to row t mod page of page
  // block_table[t / page], page = 1 << page_shift
  int paged;
  const int32_t* block_table;
  uint32_t n_blocks, num_pages, page_shift;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

// Anchor streams of coded-anchor blobs (payload rows 2L .. 4L-1) back to i8
// anchors [2][L][ng][C] at each chunk's `out`.
struct AncChunk {
  const uint8_t* blob;
  uint32_t blob_bytes;
  int32_t ng;
  uint32_t off_len, off_pay, W;
  int8_t* out;
};
struct AnchorDecodeArgs {
  int L, C, nblk, nchunks;
  AncChunk chunks[kDecMaxChunks];
  const uint16_t* afreq;  // [2][L][256]
  uint32_t* status;       // bit 0: a corrupt stream
};
hipError_t launch_anchor_decode(const AnchorDecodeArgs& a, hipStream_t st);

}  // namespace cg
