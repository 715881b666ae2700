// Internal definitions of libcachegen shared by every part: container layouts,
// format constants, conversions, the decoder's launcher.  The table builder's
// and encoder's own definitions are in cg_build.h.  Device code targets gfx950
// (wave64, 160 KB LDS per CU).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cachegen.h"

namespace cg {

// ----------------------------------------------------------------------------
// Format constants
// ----------------------------------------------------------------------------
constexpr int kNSym = 64;              // delta symbols -32..31 stored as 0..63
constexpr int kProbBits = 15;          // frequencies sum to 2^15
constexpr uint32_t kProbTotal = 1u << kProbBits;
constexpr uint32_t kTop = 1u << 24;    // range coder renormalises below 2^24
constexpr int kTabHdr = 80;
constexpr int kBlobHdr = 64;
constexpr uint32_t kTabMagic = 0x31544743u;   // "CGT1"
constexpr uint32_t kBlobMagic = 0x314B4743u;  // "CGK1"
constexpr uint32_t kBlobVersion = 2;           // payload blocks interleaved unit by unit
constexpr uint32_t kUnitWords = 4;             // a 16-byte unit of a stream
constexpr int kMaxTokens = 1 << 21;
constexpr int kMaxChunk = 65536;
constexpr int kIdLeaf = 1024;          // tables id: FNV-1a-64 tree over 1 KiB leaves,
constexpr int kIdFan = 256;            // 256 leaf digests per middle digest
constexpr int kImgRows = kNSym + 1;    // cumulative table cum[0..64]
constexpr int kLanes = 64;             // one wave64 = 64 channels
constexpr uint32_t kBufRsrcWord3 = 0x00020000u;  // raw buffer, gfx9 family

// Serialized tables: header, scale_a, inv_a, then per quality in the mask:
// step, inv_step, freq[64] — all per (kv, layer, channel).
struct TabLayout {
  size_t n = 0;  // 2 * L * C
  size_t off_scale_a = 0, off_inv_a = 0;
  size_t off_step[3] = {0, 0, 0}, off_inv_step[3] = {0, 0, 0}, off_freq[3] = {0, 0, 0};
  size_t total = 0;
  int nq = 0;
  int qslot[3] = {-1, -1, -1};  // index of quality q among the built ones
};

inline TabLayout tab_layout(int L, int C, uint32_t mask) {
  TabLayout t;
  t.n = (size_t)2 * L * C;
  size_t off = kTabHdr;
  t.off_scale_a = off;
  off += 4 * t.n;
  t.off_inv_a = off;
  off += 4 * t.n;
  for (int q = 0; q < 3; q++) {
    if (!((mask >> q) & 1)) continue;
    t.qslot[q] = t.nq++;
    t.off_step[q] = off;
    off += 4 * t.n;
    t.off_inv_step[q] = off;
    off += 4 * t.n;
    t.off_freq[q] = off;
    off += 2 * kNSym * t.n;
  }
  t.total = off;
  return t;
}

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Chunk blob: header, u32 row_offset[2][L], i8 anchors[2][L][ng][C],
// u16 lengths[2][L][C] (words), pad to 16, u32 payload[W], >= 16 zero bytes.
struct BlobLayout {
  size_t off_rows, off_anchor, off_len, off_pay;
};

inline BlobLayout blob_layout(int L, int C, int ng) {
  BlobLayout b;
  b.off_rows = kBlobHdr;
  b.off_anchor = b.off_rows + 8 * (size_t)L;
  b.off_len = b.off_anchor + 2 * (size_t)L * ng * C;
  b.off_pay = align16(b.off_len + 4 * (size_t)L * C);
  return b;
}

__host__ __device__ inline size_t blob_bytes(const BlobLayout& b, size_t W) { return align16(b.off_pay + 4 * W + 16); }

// Worst-case stream size in bytes for n symbols: each costs < 15.003 bits,
// the flush adds at most two bytes.
inline size_t stream_bytes_bound(int64_t n) {
  if (n <= 0) return 0;
  return (size_t)((n * 15 + n / 256 + 7) / 8) + 4;
}
inline size_t stream_words_bound(int64_t n) { return (stream_bytes_bound(n) + 3) / 4; }

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
  uint32_t off_anchor, off_len, off_pay, W;
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

}  // namespace cg
