// Container formats of libcachegen (serialized tables, chunk blobs) and the
// host-side checks of what callers hand in: parameters, blob headers, table
// images.  Plain C++ with no HIP dependency, so that these checks also build
// on their own (for instance under the CPU sanitizers).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

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
constexpr uint32_t kTabVersion = 1;            // tables without anchor tables
constexpr uint32_t kTabVersionCoded = 2;       // tables with one anchor table per (kv, layer)
constexpr uint32_t kBlobVersion = 2;           // raw anchors; payload blocks interleaved by unit
constexpr uint32_t kBlobVersionCoded = 3;      // the same with range-coded anchors
constexpr int kASym = 256;                     // anchor symbols: value a is a + 128
constexpr uint32_t kUnitWords = 4;             // a 16-byte unit of a stream
constexpr int kMaxTokens = 1 << 21;
constexpr int kMaxChunk = 65536;
constexpr int kIdLeaf = 1024;          // tables id: FNV-1a-64 tree over 1 KiB leaves,
constexpr int kIdFan = 256;            // 256 leaf digests per middle digest
constexpr int kImgRows = kNSym + 1;    // cumulative table cum[0..64]
constexpr int kLanes = 64;             // one wave64 = 64 channels

// Serialized tables: header, scale_a, inv_a, then per quality in the mask:
// step, inv_step, freq[64] — all per (kv, layer, channel); with coded anchors
// (version 2) then u16 afreq[2][L][256], the anchor table of each (kv, layer).
struct TabLayout {
  size_t n = 0;  // 2 * L * C
  size_t off_scale_a = 0, off_inv_a = 0;
  size_t off_step[3] = {0, 0, 0}, off_inv_step[3] = {0, 0, 0}, off_freq[3] = {0, 0, 0};
  size_t off_afreq = 0;  // 0: no anchor tables (raw anchors)
  size_t total = 0;
  int nq = 0;
  int qslot[3] = {-1, -1, -1};  // index of quality q among the built ones
};

inline TabLayout tab_layout(int L, int C, uint32_t mask, bool coded) {
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
  if (coded) {
    t.off_afreq = off;
    off += (size_t)2 * L * kASym * 2;
  }
  t.total = off;
  return t;
}

constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Chunk blob, raw anchors (version 2): header, u32 row_offset[2L], i8
// anchors[2][L][ng][C], u16 lengths[2L][C] (words), pad to 16, u32 payload[W],
// >= 16 zero bytes.  Coded anchors (version 3): header, u32 row_offset[4L],
// u16 lengths[4L][C], pad to 16, payload, >= 16 zero bytes; payload rows
// 0 .. 2L-1 are the delta streams of (kv, layer) = (r / L, r % L), rows
// 2L .. 4L-1 the anchor streams of (kv, layer) = ((r - 2L) / L, (r - 2L) % L).
struct BlobLayout {
  int rows;  // payload rows: 2L, or 4L with coded anchors
  size_t off_rows, off_anchor, off_len, off_pay;  // off_anchor 0: coded anchors
};

inline BlobLayout blob_layout(int L, int C, int ng, bool coded) {
  BlobLayout b;
  b.rows = coded ? 4 * L : 2 * L;
  b.off_rows = kBlobHdr;
  const size_t after_rows = b.off_rows + 4 * (size_t)b.rows;
  b.off_anchor = coded ? 0 : after_rows;
  b.off_len = coded ? after_rows : after_rows + 2 * (size_t)L * ng * C;
  b.off_pay = align16(b.off_len + 2 * (size_t)b.rows * C);
  return b;
}

constexpr size_t blob_bytes(const BlobLayout& b, size_t W) { return align16(b.off_pay + 4 * W + 16); }

// Worst-case stream size in bytes for n symbols: each costs < 15.003 bits,
// the flush adds at most two bytes.
inline size_t stream_bytes_bound(int64_t n) {
  if (n <= 0) return 0;
  return (size_t)((n * 15 + n / 256 + 7) / 8) + 4;
}
inline size_t stream_words_bound(int64_t n) { return (stream_bytes_bound(n) + 3) / 4; }


// ----------------------------------------------------------------------------
// Host-side checks (cg_host.cpp).  Each returns CG_OK or an error code after
// recording its message for cg_last_error().
// ----------------------------------------------------------------------------
int fail(int code, const std::string& msg);
// params with n_layer_groups = 0 replaced by the default split
int resolve_params(const cg_params* in, cg_params* out);
int check_params(const cg_params* p);
// a chunk blob's header (len bytes at b, at least the header) into o
int parse_info(const uint8_t* b, size_t len, cg_chunk_info* o);
// a serialized table image of len bytes: header, shape, every scale, step and
// frequency table the kernels rely on; its params into p
int check_tables_image(const uint8_t* b, size_t len, cg_params* p);

}  // namespace cg
