// Chunk decoder (gptget 方法详解: the receiver decodes the bitstream on the GPU;
// CacheGen blog, section 2.1: anchor plus delta reconstruction).
//
// One lane per stream (kv, layer, channel), one wave per (chunk, kv), one
// workgroup per (group of chunks with the same quality, layer, 64-channel
// block): the workgroup stages the block's 2 x 64 cumulative tables (K and V)
// in LDS once and every wave decodes its chunk's K or V streams against them.
// All lanes of a wave sit on the same token, so each reconstructed token row is
// one coalesced 128-byte store.  Blob bytes are read through a buffer resource
// bounded by the blob size: a corrupt blob reads zeros past its end instead of
// faulting.
//
// Two kernels differ only in how stream bits reach the code register:
//  * k_decode_win (workgroups of several chunks): each lane's words go through
//    an 8-word LDS ring and three symbols at a time take their bits from one
//    64-bit window of it (two v_alignbit), shifted into the code a whole byte
//    at a time with v_perm_b32;
//  * k_decode_reg (one chunk per workgroup, where the LDS holds eight
//    workgroups and so only a 4-word ring): a 64-bit register buffer refilled a
//    word at a time from the ring.
// Both level the waves' progress with s_setprio: a SIMD issues from its oldest
// ready wave first, so waves dispatched later fall behind and finish with few
// waves left to hide the LDS latency; a wave that has done more of its groups
// steps its priority down.
#include "cg_internal.h"

#include <type_traits>

namespace cg {
namespace {

__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

__device__ __forceinline__ int ld8s(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (int)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cache policy of the fp16 output stores: non-temporal.  The decoded rows are
// written once and not read back here; streaming them past the L2 leaves it to
// the lanes' stream bytes, which are re-read 8 or 16 bytes at a time.
constexpr int kStoreNT = 2;

// a ring block of RB (2 or 4) words
template <int RB>
struct Block;
template <>
struct Block<2> {
  u32x2 v;
  __device__ static Block load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return {__builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0)};
  }
};
template <>
struct Block<4> {
  u32x4 v;
  __device__ static Block load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return {__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0)};
  }
};

// The kernels' LDS is all dynamic, so it starts at LDS address 0: pointers are
// formed from byte addresses directly (constant parts of an address then fold
// into the instructions' offset fields).
template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_at(uint32_t byte_addr) {
  return reinterpret_cast<__attribute__((address_space(3))) T*>(static_cast<uintptr_t>(byte_addr));
}

__device__ __forceinline__ uint32_t lds32(uint32_t addr) { return *lds_at<uint32_t>(addr); }
__device__ __forceinline__ uint32_t lds16(uint32_t addr) { return *lds_at<uint16_t>(addr); }

// (float)((x >> 8) & 0xFF) in one instruction
__device__ __forceinline__ float byte1_to_float(uint32_t x) {
  float f;
  asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(x));
  return f;
}

// Binary16 bits (in the low half) of the value nearest to the exact a * b + c,
// ties to even: v_fma_mixlo_f16 with binary32 sources rounds the exact result
// once, to binary16.
__device__ __forceinline__ uint32_t fma_to_half(float a, float b, float c) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[0,0,0]" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// A delta token: the binary16 nearest to ahat + (s - 32) step, s being bits
// 8..13 of the symbol's LDS address (s - 32 is exact in binary32).
__device__ __forceinline__ uint32_t delta_half(uint32_t ad, float step, float ahat) {
  return fma_to_half(byte1_to_float(ad) - 32.0f, step, ahat);
}

// The workgroup's LDS holds the K and V tables of one (layer, 64-channel block)
// side by side: row k = [cum[k] of the 64 K streams | cum[k] of the 64 V
// streams], 256 bytes, so the byte address of entry k of a lane is
// k * 256 + (kv * 128 + 2 * slot) and bits 8..15 of it are k itself.
constexpr uint32_t kRow = 4 * kLanes;
constexpr uint32_t kTabBytes = kImgRows * kRow;        // 16,640
constexpr uint32_t kSlot = 4 * kLanes;                 // a ring slot: one word per lane

// All ones when r * key <= code, else zero.  ncode is ~code, so the 64-bit sum
// r * key + (2^64 - code - 1) stays within [2^64 - 2^32, 2^64) when
// r * key <= code and otherwise wraps to r * key - code - 1 < 2^32: its high
// word is the mask (one v_mad_u64_u32; r * key < 2^32).
__device__ __forceinline__ uint32_t le_mask(uint32_t r, uint32_t key, uint32_t ncode) {
  const uint64_t c = 0xFFFFFFFF00000000ull | ncode;
  return (uint32_t)(((uint64_t)r * key + c) >> 32);
}

// (m & a) | (~m & b) as one v_bfi_b32 (left to itself the compiler picks
// v_bitop3_b32, which a miscompiled decoder variant used on the result of the
// v_mad_u64_u32 just before it)
__device__ __forceinline__ uint32_t bit_select(uint32_t m, uint32_t a, uint32_t b) {
  uint32_t d;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(d) : "v"(m), "v"(a), "v"(b));
  return d;
}

// The lanes in which a + b carries out of 32 bits, as a wave mask (one
// v_add_co_u32 with its carry in a scalar register pair)
__device__ __forceinline__ uint64_t carry_mask(uint32_t a, uint32_t b) {
  uint32_t sum;
  uint64_t c;
  asm("v_add_co_u32 %0, %1, %2, %3" : "=v"(sum), "=s"(c) : "v"(a), "v"(b));
  return c;
}

// One symbol's search and interval update.  Returns the LDS address of
// cum[s] (bits 8..13 are s); leaves ncode = ~(code - r cum[s]) and range =
// r freq[s] shifted left by sh bits, sh = 0, 8 or 16 (whole bytes until range
// >= 2^24; r freq >= 2^9), and the caller shifts sh stream bits into ncode.
//
// s is the largest symbol with r cum[s] <= code.  Delta symbols crowd around
// the zero delta (symbol 32), so the search first bisects the 16 symbols
// [24, 40) only: the root cum[32] and the second level's cum[28] and cum[36]
// are in registers, then two levels from LDS.  The result is the answer
// exactly when code - r cum[s] lies in [0, r freq[s]), i.e. when
// ~(code - r cum[s]) + r freq[s] carries out of 32 bits; a lane whose symbol
// lies outside the window (or whose stream is corrupt) fails that test, and
// then the wave redoes the symbol with the full six-level bisection (valid
// lanes find the same symbol again).
__device__ __forceinline__ uint32_t search(uint32_t& ncode, uint32_t& range, uint32_t& sh,
                                           uint32_t lane_addr, uint32_t key32, uint32_t key28,
                                           uint32_t key36) {
  const uint32_t r = range >> kProbBits;
  const uint32_t m = le_mask(r, key32, ncode);
  // cum[32] <= code: window [32, 40), else [24, 32); its middle key is in a
  // register too
  const uint32_t m2 = le_mask(r, bit_select(m, key36, key28), ncode);
  uint32_t ad = bit_select(m, lane_addr + 32u * kRow, lane_addr + 24u * kRow) | (m2 & (4u * kRow));
#pragma unroll
  for (uint32_t stp = 2; stp; stp >>= 1) ad |= le_mask(r, lds16(ad + stp * kRow), ncode) & (stp * kRow);
  uint32_t c0 = lds16(ad), c1 = lds16(ad + kRow);
  uint32_t nc2 = ncode + mul24(r, c0);  // code -= r * cum[s]
  uint32_t rn = mul24(r, c1 - c0);
  // no carry in some lane: redo the whole wave with the full search (a
  // wave-uniform branch, laid out away from the common path)
  if (__builtin_expect(carry_mask(nc2, rn) != __builtin_amdgcn_read_exec(), 0)) {
    ad = lane_addr | (m & (32u * kRow));
#pragma unroll
    for (uint32_t stp = 16; stp; stp >>= 1) ad |= le_mask(r, lds16(ad + stp * kRow), ncode) & (stp * kRow);
    c0 = lds16(ad);
    c1 = lds16(ad + kRow);
    nc2 = ncode + mul24(r, c0);
    rn = mul24(r, c1 - c0);
  }
  ncode = nc2;
  sh = (uint32_t)__builtin_clz(rn) & 24u;
  range = rn << sh;
  return ad;
}

// v_perm_b32 selector that picks the high word of {hi:lo} << sh (sh = 0, 8, 16
// or 24): byte i of the result is byte i + 4 - sh / 8 of the pair
__device__ __forceinline__ uint32_t shift_sel(uint32_t sh) {
  return (uint32_t)((0x0706050403020100ull << sh) >> 32);
}

// Where a lane's stream lies in the payload layout.  A 64-stream block holds
// m whole 16-byte units of every one of its ns streams first, unit by unit,
// then each stream's remaining words: word w of the lane's stream is at byte
// a0 + (w / 4) us + 4 (w % 4) while w / 4 < m (us = 16 ns bytes between the
// units of one stream), else at t0 + 4 w (t0 = where its tail starts, less
// 16 m).  m and us are the same for the whole wave.
struct Words {
  uint32_t a0, t0, us, m;
  // byte offset of unit u (words 4u .. 4u + 3)
  __device__ __forceinline__ uint32_t unit(uint32_t u) const {
    const uint32_t inter = a0 + mul24(u, us), tail = t0 + (u << 4);
    return u < m ? inter : tail;
  }
  __device__ __forceinline__ uint32_t word(uint32_t w) const { return unit(w >> 2) + 4u * (w & 3u); }
};

// Per-lane state both kernels set up the same way.
struct Lane {
  __amdgpu_buffer_rsrc_t rs, ro;
  __amdgpu_buffer_rsrc_t ra;  // the chunk's anchors
  Words wd;            // the lane's stream words in the blob
  uint32_t bad;        // stream extends past the payload
  float scale_a, step;
  uint32_t lane_addr;  // LDS address of the lane's cum[0]
  uint32_t key32;      // cum[32], the root of every search
  uint32_t key28, key36;  // cum[28] and cum[36], the keys of its second level
  uint32_t row_bytes, lane_off, anc_base;
  int C;
  DecChunk ch;
  // paged output: the layer's pool, its size in bytes, the block table and the
  // chunk's first context token
  uint16_t* pool;
  uint32_t pool_bytes;
  __amdgpu_buffer_rsrc_t rt;
  uint32_t tok0;
};

// Words of the streams of a row's 64-channel blocks before block cb: the sum
// of their u16 lengths at len_base, summed over the wave (every lane gets the
// total).  Four loads in flight per lane; an index past them points past the
// blob's end (no memory access).
__device__ __forceinline__ uint32_t words_before(__amdgpu_buffer_rsrc_t rs, uint32_t len_base,
                                                 int cb, int lane) {
  const uint32_t n = (uint32_t)(cb * kLanes);
  uint32_t before = 0;
  for (uint32_t j = (uint32_t)lane; j < n; j += 4u * kLanes) {
    uint32_t q[4];
#pragma unroll
    for (uint32_t i = 0; i < 4; i++) {
      const uint32_t jj = j + i * kLanes;
      q[i] = ld16(rs, jj < n ? len_base + 2u * jj : 0xFFFFFFF0u);
    }
    before += q[0] + q[1] + q[2] + q[3];
  }
  for (int o = 32; o; o >>= 1) before += __shfl_xor(before, o);
  return before;
}

// The warming wave of a workgroup: reads one word of every 64 bytes of the
// block's streams of each chunk and kv (a contiguous byte range of the blob;
// its first 64 KB), 16 loads in flight at a time.  A lane fetches its stream
// 16 bytes at a time and needs the rest of a cache line only several groups
// later, when the line has often left the L2; read ahead of the decoding waves
// by a wave of its own (whose waits do not hold them up), the lines are served
// by the memory-side cache instead of HBM.  Loads past a range point past the
// blob's end (no memory access).
__device__ __forceinline__ void warm_block(const DecodeArgs& a, int grp, int l, int cb, int lane) {
  uint32_t x = 0;
  for (int w = 0; w < 4; w++) {
    const int ci = a.groups[grp].chunk[w];
    if (ci < 0) continue;
    const DecChunk ch = a.chunks[ci];
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)ch.blob, 0, (int)ch.blob_bytes, kBufRsrcWord3);
    for (int kv = 0; kv < 2; kv++) {
      const int row = kv * a.L + l;
      const uint32_t len_base = ch.off_len + 2u * (uint32_t)row * (uint32_t)a.C;
      const uint32_t before = words_before(rs, len_base, cb, lane);
      const int c = cb * kLanes + lane;
      uint32_t mine = c < a.C ? ld16(rs, len_base + 2u * c) : 0u;
      for (int o = 32; o; o >>= 1) mine += __shfl_xor(mine, o);
      const uint32_t start = ld32(rs, 64u + 4u * row) + before;  // words into the payload
      const uint32_t lo = (ch.off_pay + 4u * start) & ~63u;
      const uint32_t hi = ch.off_pay + 4u * (start + mine);
      const uint32_t n = __builtin_amdgcn_readfirstlane(hi > lo ? (hi - lo + 4095u) >> 12 : 0u);
#pragma unroll
      for (uint32_t k = 0; k < 16; k++)
        x ^= ld32(rs, k < n ? lo + (k << 12) + 64u * (uint32_t)lane : 0xFFFFFFF0u);
    }
  }
  if (x & a.sink_mask) atomicOr(a.status, 4u);
}

// Stages the tables and sets up the lane; false for a lane without a stream
// (and for the warming wave, after its reads).
template <bool PG>
__device__ __forceinline__ bool setup(const DecodeArgs& a, int wave, int lane, Lane& s) {
  auto tab = lds_at<uint32_t>(0);
  const int tid = threadIdx.x;
  const int per_grp = a.L * a.nblk;
  const int grp = blockIdx.x / per_grp, rem = blockIdx.x % per_grp;
  const int l = rem / a.nblk, cb = rem % a.nblk;
  const int q = a.chunks[a.groups[grp].chunk[0]].q;
  {
    constexpr size_t img_u32 = kImgRows * kLanes / 2;
    const uint32_t* src_k = reinterpret_cast<const uint32_t*>(a.img[q]) +
                            ((size_t)l * a.nblk + cb) * img_u32;
    const uint32_t* src_v = reinterpret_cast<const uint32_t*>(a.img[q]) +
                            ((size_t)(a.L + l) * a.nblk + cb) * img_u32;
    for (int j = tid; j < kImgRows * kLanes; j += blockDim.x) {
      const int row = j >> 6, half = (j >> 5) & 1, w = j & 31;
      tab[j] = (half ? src_v : src_k)[row * 32 + w];
    }
  }
  __syncthreads();
  if (a.warm_wave && wave == 2 * a.waves) {
    warm_block(a, grp, l, cb, lane);
    return false;
  }
  const int kv = wave & 1;
  const int ci = a.groups[grp].chunk[wave >> 1];
  if (ci < 0) return false;
  s.ch = a.chunks[ci];
  s.rs = __builtin_amdgcn_make_buffer_rsrc((void*)s.ch.blob, 0, (int)s.ch.blob_bytes, kBufRsrcWord3);
  const int row = kv * a.L + l;
  const int c = cb * kLanes + lane;
  const bool active = c < a.C;

  // the block's place in the payload (row offset + the words of the row's
  // earlier blocks), its units m and the lane's tail offset (the whole wave
  // takes part in the reductions and the scan)
  const uint32_t len_base = s.ch.off_len + 2u * (uint32_t)row * (uint32_t)a.C;
  const uint32_t before = words_before(s.rs, len_base, cb, lane);
  const uint32_t my_len = active ? ld16(s.rs, len_base + 2u * c) : 0u;
  uint32_t total = my_len, mu = active ? my_len >> 2 : 0xFFFFFFFFu;
  for (int o = 32; o; o >>= 1) {
    total += __shfl_xor(total, o);
    mu = min(mu, __shfl_xor(mu, o));
  }
  const uint32_t m = __builtin_amdgcn_readfirstlane(mu);
  const uint32_t ns = (uint32_t)min(kLanes, a.C - cb * kLanes);
  const uint32_t tl = active ? my_len - 4u * m : 0u;  // the lane's tail words
  uint32_t incl = tl;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (!active) return false;  // no cross-lane work after this
  const uint32_t blk = ld32(s.rs, 64u + 4u * row) + before;  // words into the payload
  s.bad = ((uint64_t)blk + total > s.ch.W) ? 1u : 0u;
  const uint32_t blk_byte = s.ch.off_pay + 4u * blk;
  s.wd.m = m;
  s.wd.us = 16u * ns;
  s.wd.a0 = blk_byte + 16u * (uint32_t)lane;
  s.wd.t0 = blk_byte + 4u * (4u * m * ns + incl - tl) - 16u * m;

  const size_t pi = (size_t)row * a.C + c;
  s.scale_a = a.scale_a[pi];
  s.step = a.step[q][pi];
  s.lane_addr = (uint32_t)kv * (2u * kLanes) + 2u * lane_slot(lane);
  s.key32 = lds16(s.lane_addr + 32u * kRow);
  s.key28 = lds16(s.lane_addr + 28u * kRow);
  s.key36 = lds16(s.lane_addr + 36u * kRow);

  // output rows of this (kv, layer, chunk) through a buffer resource: the lane's
  // channel is the vector offset, the token row a wave-uniform scalar offset
  if constexpr (PG) {
    const size_t layer_elems = ((size_t)a.num_pages << a.page_shift) * (size_t)a.C;
    s.pool = (kv ? a.v_out : a.k_out) + (size_t)l * layer_elems;
    s.pool_bytes = (uint32_t)(2u * layer_elems);
    s.rt = __builtin_amdgcn_make_buffer_rsrc((void*)a.block_table, 0, (int)(4u * a.n_blocks),
                                             kBufRsrcWord3);
    s.tok0 = (uint32_t)s.ch.t0;
  } else {
    uint16_t* const out_base = (kv ? a.v_out : a.k_out) + ((size_t)l * a.T + s.ch.t0) * a.C;
    s.ro = __builtin_amdgcn_make_buffer_rsrc(out_base, 0, (int)((uint32_t)s.ch.tc * (uint32_t)a.C * 2u),
                                             kBufRsrcWord3);
  }
  s.row_bytes = 2u * (uint32_t)a.C;
  s.lane_off = 2u * (uint32_t)c;
  s.ra = __builtin_amdgcn_make_buffer_rsrc((void*)s.ch.anc, 0, (int)s.ch.anc_bytes, kBufRsrcWord3);
  s.anc_base = (uint32_t)row * (uint32_t)s.ch.ng * (uint32_t)a.C + c;
  s.C = a.C;
  return true;
}

// stores the binary16 in the low half of h as token row t of the lane's channel
__device__ __forceinline__ void put_half(const Lane& s, uint32_t h, uint32_t t) {
  __builtin_amdgcn_raw_buffer_store_b16((uint16_t)h, s.ro, s.lane_off, t * s.row_bytes, kStoreNT);
}

// ---------------------------------------------------------------------------
// Paged output.  Lane j of a wave holds the byte offset, in the layer's pool,
// of the row of token j of the current group (groups are at most 64 tokens),
// computed from the block-table entry it loaded one group earlier; a token's
// store reads it with one v_readlane.  An entry outside the pool gives kNoRow:
// that row's stores get a resource of size zero, so they write nothing.
constexpr uint32_t kNoRow = 0xFFFFFFFFu;

struct Pager {
  uint32_t po = 0;    // this lane's token row offset in the current group, or kNoRow
  uint32_t ent = 0;   // block-table entry of this lane's token in the next group (in flight)
  uint32_t bad = 0;   // an entry this lane needed was outside the pool
  int ta = 0;         // first token (in the chunk) of the current group

  // issues the load of the entry for token ta + lane (lanes past the group
  // point their load past the table: no memory access, zero)
  __device__ __forceinline__ void fetch(const DecodeArgs& a, const Lane& s, int lane, int ta_next) {
    const uint32_t tok = s.tok0 + (uint32_t)ta_next + (uint32_t)lane;
    ent = ld32(s.rt, lane < a.G ? 4u * (tok >> a.page_shift) : 0xFFFFFFF0u);
  }
  // the current group [ta, te) takes the entries fetched for it
  __device__ __forceinline__ void begin(const DecodeArgs& a, const Lane& s, int lane, int ta_, int te) {
    ta = ta_;
    const uint32_t tok = s.tok0 + (uint32_t)ta + (uint32_t)lane;
    const bool ok = ent < a.num_pages;
    if (!ok && lane < te - ta) bad = 1u;
    po = ok ? ((ent << a.page_shift) | (tok & ((1u << a.page_shift) - 1u))) * s.row_bytes : kNoRow;
  }
  __device__ __forceinline__ void put(const Lane& s, uint32_t h, uint32_t t) const {
    const uint32_t ro = (uint32_t)__builtin_amdgcn_readlane((int)po, (int)t - ta);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(s.pool, 0, ro != kNoRow ? (int)s.pool_bytes : 0, kBufRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)h, r, s.lane_off, ro, kStoreNT);
  }
};

// ---------------------------------------------------------------------------
// LDS-window kernel.  Per lane, ring word k (stream word 1 + k) sits,
// complemented, in slot 2 + M - (k mod 8) (M = 7: later words in lower slots)
// and slots 1 and 0 repeat the words with k mod 8 = 0 and 1, so words j, j + 1,
// j + 2 are always the three consecutive slots s + 2, s + 1, s with
// s = M - (j mod 8).  Blocks of four words land once per group, fetched one
// group ahead.
constexpr int kWinRB = 4;
constexpr uint32_t kWinM = 2u * kWinRB - 1u;
__host__ __device__ constexpr uint32_t win_ring_bytes() { return (2u * kWinRB + 2u) * kSlot; }

// a block's words, complemented, into their slots.  A block starts at a ring
// index that is 0 or 4 mod 8, so it fills slots 6..9 ("high": its first two
// words are also repeated in slots 1 and 0) or slots 2..5; at = the byte
// address of its lowest slot.
__device__ __forceinline__ void win_put(uint32_t ring, uint32_t at, bool high, const Block<kWinRB>& b) {
  auto p = lds_at<uint32_t>(at);
  const uint32_t w0 = ~b.v.x, w1 = ~b.v.y, w2 = ~b.v.z, w3 = ~b.v.w;
  p[3 * kLanes] = w0;
  p[2 * kLanes] = w1;
  p[kLanes] = w2;
  p[0] = w3;
  if (high) {
    auto m = lds_at<uint32_t>(ring);
    m[kLanes] = w0;
    m[0] = w1;
  }
}
constexpr uint32_t kWinHigh = (2u + kWinM - (kWinRB - 1u)) * kSlot;  // lowest slot of a high block
constexpr uint32_t kWinLow = kWinHigh - kWinRB * kSlot;

template <int GS, bool PG>
__global__ __launch_bounds__(512) void k_decode_win(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Lane s;
  if (!setup<PG>(a, wave, lane, s)) return;
  Pager pg;
  auto out = [&](uint32_t t, uint32_t h) {
    if constexpr (PG) pg.put(s, h, t);
    else put_half(s, h, t);
  };
  constexpr int RB = kWinRB;
  constexpr uint32_t M = kWinM;

  // decoder state: ncode = ~code, range, and nc = -(32 + stream bits shifted
  // into the code after its first word): ring word k is stream word k, so the
  // next bits start 32 + those bits into the ring
  const Block<RB> b0 = Block<RB>::load(s.rs, s.wd.unit(0));
  const Block<RB> b1 = Block<RB>::load(s.rs, s.wd.unit(1));
  uint32_t ncode = ~b0.v.x;
  uint32_t range = 0xFFFFFFFFu;
  uint32_t nc = (uint32_t)-32;
  const uint32_t ring = kTabBytes + (uint32_t)wave * win_ring_bytes() + 4u * (uint32_t)lane;
  // Ring words 0 .. n - 1 have been written, n = (64 - lim) / 32: nc < lim
  // means a window's words have not all landed.  fetched = the words fetched,
  // landed or in flight (the next block holds unit fetched / 4); land = where
  // the next block lands (the high and low halves alternate, so land toggles
  // as flip - land).
  int lim = 64 - 32 * (int)(2u * RB);
  uint32_t fetched = 2u * RB;
  const uint32_t flip = 2u * ring + kWinHigh + kWinLow;
  uint32_t land = ring + kWinHigh;
  win_put(ring, ring + kWinHigh, true, b0);
  win_put(ring, ring + kWinLow, false, b1);
  Block<RB> pend = {};  // block in flight
  bool inflight = false;
  int anc_next = ld8s(s.ra, s.anc_base);

  // one symbol, its new bits x (the next stream bits, most significant first);
  // returns sh and the selector that shifted them in
  auto symbol = [&](uint32_t t, float ahat, uint32_t x, uint32_t& sel) -> uint32_t {
    uint32_t sh;
    const uint32_t ad = search(ncode, range, sh, s.lane_addr, s.key32, s.key28, s.key36);
    sel = shift_sel(sh);
    ncode = __builtin_amdgcn_perm(ncode, x, sel);
    out(t, delta_half(ad, s.step, ahat));
    return sh;
  };

  // N (1..3) symbols from one 64-bit window of the stream (they take at most
  // 48 bits)
  auto run = [&](auto n_c, uint32_t t, float ahat) {
    constexpr int N = decltype(n_c)::value;
    if ((int)nc < lim) {
      // the ring has run dry (more bits taken than fetched, which typical data
      // never does): the missing words straight from the blob
      const uint32_t j = ~nc >> 5;
      int l = lim;
      asm volatile("" : "+v"(l));  // computed here, not in every group
      const uint32_t landed = (uint32_t)(64 - l) >> 5;
#pragma unroll
      for (uint32_t d = 0; d < 3; d++) {
        const uint32_t k = j + d;
        if (k >= landed) {
          const uint32_t w = ~ld32(s.rs, s.wd.word(k));
          const uint32_t sl = k & M;
          *lds_at<uint32_t>(ring + (2u + M - sl) * kSlot) = w;
          if (sl < 2u) *lds_at<uint32_t>(ring + (1u - sl) * kSlot) = w;
        }
      }
    }
    // words j, j + 1, j + 2 with j = ceil(bits / 32) - 1: the window starts
    // (-bits) mod 32 bits into word j
    uint32_t sl = __builtin_amdgcn_ubfe(nc, 5u, 3u);
    asm volatile("" : "+v"(sl));  // keeps the address one shift-add of the slot
    const uint32_t ba = ring + (sl << 8);
    const uint32_t w0 = lds32(ba + 2u * kSlot), w1 = lds32(ba + kSlot), w2 = lds32(ba);
    const uint32_t hi = __builtin_amdgcn_alignbit(w0, w1, nc);
    const uint32_t lo = __builtin_amdgcn_alignbit(w1, w2, nc);
    uint32_t sel1, sel2, sel3;
    uint32_t tot = symbol(t, ahat, hi, sel1);
    if constexpr (N >= 2) {
      const uint64_t win = (((uint64_t)hi << 32) | lo) << tot;
      const uint32_t h2 = (uint32_t)(win >> 32), l2 = (uint32_t)win;
      const uint32_t sh2 = symbol(t + 1, ahat, h2, sel2);
      tot += sh2;
      if constexpr (N >= 3) tot += symbol(t + 2, ahat, __builtin_amdgcn_perm(h2, l2, sel2), sel3);
    }
    nc -= tot;
  };

  // once per group: write the block fetched one group earlier into the ring,
  // then fetch the next unit if the words it lands over are taken (lanes
  // without room point their load past the blob end: no memory access)
  auto ring_step = [&]() {
    if (inflight) {
      win_put(ring, land, land == ring + kWinHigh, pend);
      land = flip - land;
      lim -= 32 * RB;
    }
    inflight = (int)nc <= 64 - 32 * (int)fetched + 32 * RB - 64;
    pend = Block<RB>::load(s.rs, inflight ? s.wd.unit(fetched >> 2) : 0xFFFFFFF0u);
    fetched += inflight ? (uint32_t)RB : 0u;
  };

  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  auto group = [&](int g, int ta, int te) {
    ring_step();
    if constexpr (PG) {
      pg.begin(a, s, lane, ta, te);
      pg.fetch(a, s, lane, ta + (GS > 0 ? GS : a.G));
    }
    const int anc = anc_next;
    anc_next = ld8s(s.ra, s.anc_base + (uint32_t)(g + 1) * s.C);  // past the last group: unused
    const float ahat = anchor_value(anc, s.scale_a);
    out((uint32_t)ta, float_to_half_bits(ahat));
    int t = ta + 1;
#pragma unroll
    for (; t + 2 < te; t += 3) {
      __builtin_amdgcn_sched_barrier(0);
      run(I3{}, (uint32_t)t, ahat);
    }
    if (t + 1 < te) {
      __builtin_amdgcn_sched_barrier(0);
      run(I2{}, (uint32_t)t, ahat);
    } else if (t < te) {
      __builtin_amdgcn_sched_barrier(0);
      run(I1{}, (uint32_t)t, ahat);
    }
  };

  // everything loaded so far (scale, step, first words, first anchor) is in
  // registers before the loop, so no wait inside it is for those loads
  if constexpr (PG) pg.fetch(a, s, lane, 0);
  __builtin_amdgcn_s_waitcnt(0);
  // Full groups of the compile-time size GS run the same unrolled code, and a
  // wave's priority steps 3 -> 2 -> 1 -> 0 at half, three quarters and seven
  // eighths of them; the rest (a last partial group, or every group when
  // GS = 0) follow at the priority reached.
  int g = 0;
  if constexpr (GS > 0) {
    const int nfull = s.ch.tc / GS;
    const int q1 = nfull >> 1, q2 = nfull - (nfull >> 2), q3 = nfull - (nfull >> 3);
    __builtin_amdgcn_s_setprio(3);
    for (; g < nfull; g++) {
      if (g == q1) __builtin_amdgcn_s_setprio(2);
      if (g == q2) __builtin_amdgcn_s_setprio(1);
      if (g == q3) __builtin_amdgcn_s_setprio(0);
      group(g, g * GS, g * GS + GS);
    }
  }
  for (; g < s.ch.ng; g++) group(g, g * a.G, min(g * a.G + a.G, s.ch.tc));
  // a valid stream keeps code < range throughout; a corrupt one breaks it for good
  s.bad |= (~ncode >= range) ? 1u : 0u;
  if (s.bad) atomicOr(a.status, 1u);
  if (PG && pg.bad) atomicOr(a.status, 2u);
}

// ---------------------------------------------------------------------------
// Register-buffer kernel.  A wave's word ring: 4 slots x 64 lanes; the first
// wave's ring is aligned to the ring size, so a slot address is the lane's ring
// address with the slot number in the bits above 7.
constexpr int kRegRB = 2;
__host__ __device__ constexpr uint32_t reg_ring_bytes() { return 2u * kRegRB * kSlot; }
__host__ __device__ constexpr uint32_t reg_ring_base() {
  return (kTabBytes + reg_ring_bytes() - 1) / reg_ring_bytes() * reg_ring_bytes();
}

__device__ __forceinline__ void reg_put(uint32_t lane_addr, uint32_t slot_off, const Block<kRegRB>& b) {
  auto p = lds_at<uint32_t>(lane_addr + slot_off);
  p[0] = b.v.x;
  p[64] = b.v.y;
}

template <int GS, bool PG>
__global__ __launch_bounds__(512) void k_decode_reg(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Lane s;
  if (!setup<PG>(a, wave, lane, s)) return;
  Pager pg;
  auto out = [&](uint32_t t, uint32_t h) {
    if constexpr (PG) pg.put(s, h, t);
    else put_half(s, h, t);
  };
  constexpr int RB = kRegRB;

  // decoder state: ncode = ~code; range; bb = the next bits of the stream,
  // complemented, in its low `left` bits (most significant first, 32..64 of
  // them before every pair of symbols).  Words 0..2 start the state; words 3..
  // reach bb through the wave's LDS ring: word k sits in slot k mod 2 RB of the
  // lane's column, fetched RB words (half a unit) at a time one group ahead of
  // use.  Word 3 and words 4, 5 are written below.
  static_assert(kRegRB == 2, "the ring holds half units");
  const u32x4 u0 = __builtin_amdgcn_raw_buffer_load_b128(s.rs, s.wd.unit(0), 0, 0);
  const Block<RB> b1 = Block<RB>::load(s.rs, s.wd.word(4));
  uint32_t ncode = ~u0.x;
  uint64_t bb = ((uint64_t)~u0.y << 32) | ~u0.z;
  uint32_t left = 64;
  uint32_t range = 0xFFFFFFFFu;
  constexpr uint32_t kSlotMask = (2u * RB - 1u) << 8;
  const uint32_t ring = reg_ring_base() + (uint32_t)wave * reg_ring_bytes() + 4u * (uint32_t)lane;
  // words taken from the ring and written to it, counted in units of 256 (one
  // slot's size): the next word to take is word 3, words 3 .. 5 are written
  uint32_t taken = 3u << 8;
  uint32_t landed = 6u << 8;
  uint32_t fetch_w = 6;  // the next block's first word
  *lds_at<uint32_t>(ring + (3u << 8)) = u0.w;
  reg_put(ring, 0u, b1);
  Block<RB> pend = {};  // block in flight
  bool inflight = false;
  int anc_next = ld8s(s.ra, s.anc_base);

  // one symbol: search, interval update, renormalisation, reconstruction
  auto symbol = [&](uint32_t t, float ahat) {
    uint32_t sh;
    const uint32_t ad = search(ncode, range, sh, s.lane_addr, s.key32, s.key28, s.key36);
    const uint32_t tl = left - sh;
    ncode = (ncode << sh) | __builtin_amdgcn_ubfe((uint32_t)(bb >> (tl & 63u)), 0u, sh);
    left = tl;
    out(t, delta_half(ad, s.step, ahat));
  };

  // A lane takes a word when fewer than 32 bits remain (two symbols need at
  // most 32).  Only stores go to memory inside a group, so no wait in it
  // drains them; a ring that has run dry (more than the buffered words taken
  // in one group, which typical data never does) falls back to a direct load.
  auto refill = [&]() {
    const bool take = left < 32;
    const uint32_t slot = (taken & kSlotMask) | ring;
    if (take && taken >= landed)
      *lds_at<uint32_t>(slot) = ld32(s.rs, s.wd.word(taken >> 8));
    const uint32_t w = lds32(slot);
    if (take) {
      bb = (bb << 32) | ~w;
      left += 32;
      taken += 256u;
    }
  };
  // once per group: write the block fetched one group earlier into the ring,
  // then fetch the next one if the ring has room for it when it lands (lanes
  // without room point their load past the blob end: no memory access)
  auto ring_step = [&]() {
    if (inflight) {
      reg_put(ring, landed & ((uint32_t)RB << 8), pend);
      landed += (uint32_t)RB << 8;
    }
    inflight = landed + ((uint32_t)RB << 8) <= taken + ((2u * RB) << 8);
    pend = Block<RB>::load(s.rs, inflight ? s.wd.word(fetch_w) : 0xFFFFFFF0u);
    if (inflight) fetch_w += RB;
  };

  // one group: the anchor row, then its deltas in pairs (a lone last one when
  // the group has an even number of tokens)
  auto group = [&](int g, int ta, int te) {
    ring_step();
    if constexpr (PG) {
      pg.begin(a, s, lane, ta, te);
      pg.fetch(a, s, lane, ta + (GS > 0 ? GS : a.G));
    }
    const int anc = anc_next;
    anc_next = ld8s(s.ra, s.anc_base + (uint32_t)(g + 1) * s.C);  // past the last group: unused
    const float ahat = anchor_value(anc, s.scale_a);
    out((uint32_t)ta, float_to_half_bits(ahat));
    int t = ta + 1;
#pragma unroll
    for (; t + 1 < te; t += 2) {
      // keep the refill after the previous pair's stores: its wait then
      // leaves those two stores in flight
      __builtin_amdgcn_sched_barrier(0);
      refill();
      symbol((uint32_t)t, ahat);
      symbol((uint32_t)(t + 1), ahat);
    }
    if (t < te) {
      __builtin_amdgcn_sched_barrier(0);
      refill();
      symbol((uint32_t)t, ahat);
    }
  };

  if constexpr (PG) pg.fetch(a, s, lane, 0);
  __builtin_amdgcn_s_waitcnt(0);
  // Full groups of the compile-time size GS run the same unrolled code, and a
  // wave's priority steps 3 -> 2 -> 1 -> 0 at half, three quarters and seven
  // eighths of them; the rest (a last partial group, or every group when
  // GS = 0) follow at the priority reached.
  int g = 0;
  if constexpr (GS > 0) {
    const int nfull = s.ch.tc / GS;
    const int q1 = nfull >> 1, q2 = nfull - (nfull >> 2), q3 = nfull - (nfull >> 3);
    __builtin_amdgcn_s_setprio(3);
    for (; g < nfull; g++) {
      if (g == q1) __builtin_amdgcn_s_setprio(2);
      if (g == q2) __builtin_amdgcn_s_setprio(1);
      if (g == q3) __builtin_amdgcn_s_setprio(0);
      group(g, g * GS, g * GS + GS);
    }
  }
  for (; g < s.ch.ng; g++) group(g, g * a.G, min(g * a.G + a.G, s.ch.tc));
  s.bad |= (~ncode >= range) ? 1u : 0u;
  if (s.bad) atomicOr(a.status, 1u);
  if (PG && pg.bad) atomicOr(a.status, 2u);
}

// ---------------------------------------------------------------------------
// Anchor streams of coded-anchor blobs.  One lane per stream (kv, layer,
// channel) of a chunk, one wave per 64-channel block, a workgroup per (four
// blocks, (kv, layer), chunk) sharing the (kv, layer) anchor table's cumulative
// counts in LDS.  A lane
// reads its stream through the payload layout (as the delta decoders do) and
// writes anchor s - 128 of every group to the chunk's anchor array, 64 bytes
// per wave and group.
//
// Symbols go in rounds of eight, wave-uniform like the delta decoders' groups:
// at the end of a round a lane lands the 16-byte unit it fetched one round
// earlier into its 16-word LDS ring and fetches the next unit if the ring has
// room, so no wait inside a round is for memory, and every wait for a unit
// comes after the same eight stores (an exact count).  A symbol takes at most
// 16 bits (r freq >= 2^9), a round at most 128: one unit per round keeps up,
// and a lead of two units (the ring starts with two landed) always covers the
// round's windows.  Two symbols at a time take their bits from one 64-bit
// window (three ring words); the symbol is the largest s with r cum[s] <= code,
// found by an eight-level bisection (each level one v_mad_u64_u32 mask, as in
// the delta search); the code is held complemented, shifted a whole byte at a
// time with v_perm_b32.
constexpr uint32_t kAncRing = 16;  // ring words per lane
constexpr int kAncRound = 8;       // symbols per round
constexpr int kAncWaves = 4;       // blocks (waves) per workgroup
// dynamic LDS (from address 0): cum[0..256], then a ring [16 slots][64 lanes]
// per wave
constexpr uint32_t kAncRingAt = 4u * (kASym + 4);
constexpr uint32_t kAncRingBytes = 4u * kAncRing * kLanes;
constexpr uint32_t kAncLds = kAncRingAt + kAncWaves * kAncRingBytes;

__global__ __launch_bounds__(64 * kAncWaves) void k_anchor_decode(AnchorDecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto cum = lds_at<uint32_t>(0);
  auto ring = lds_at<uint32_t>(kAncRingAt + (uint32_t)wave * kAncRingBytes);
  const int cb = blockIdx.x * kAncWaves + wave, arow = blockIdx.y;  // arow = kv * L + l
  const AncChunk ch = a.chunks[blockIdx.z];
  if (wave == 0) {
    const uint16_t* f = a.afreq + (size_t)arow * kASym + 4 * lane;
    const uint32_t f0 = f[0], f1 = f[1], f2 = f[2], f3 = f[3];
    uint32_t incl = f0 + f1 + f2 + f3;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const uint32_t base = incl - (f0 + f1 + f2 + f3);
    cum[4 * lane] = base;
    cum[4 * lane + 1] = base + f0;
    cum[4 * lane + 2] = base + f0 + f1;
    cum[4 * lane + 3] = base + f0 + f1 + f2;
    if (lane == 63) cum[kASym] = incl;
  }
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)ch.blob, 0, (int)ch.blob_bytes, kBufRsrcWord3);
  const int prow = 2 * a.L + arow;  // the payload row of these streams
  const int c = cb * kLanes + lane;
  const bool active = c < a.C;
  // the stream's words in the payload layout, as in the delta decoders' setup
  const uint32_t len_base = ch.off_len + 2u * (uint32_t)prow * (uint32_t)a.C;
  const uint32_t before = words_before(rs, len_base, cb, lane);
  const uint32_t my_len = active ? ld16(rs, len_base + 2u * c) : 0u;
  uint32_t total = my_len, mu = active ? my_len >> 2 : 0xFFFFFFFFu;
  for (int o = 32; o; o >>= 1) {
    total += __shfl_xor(total, o);
    mu = min(mu, __shfl_xor(mu, o));
  }
  const uint32_t m = __builtin_amdgcn_readfirstlane(mu);
  const uint32_t ns = (uint32_t)min(kLanes, a.C - cb * kLanes);
  const uint32_t tl = active ? my_len - 4u * m : 0u;
  uint32_t incl = tl;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  __syncthreads();  // the cumulative table
  if (cb >= a.nblk || !active) return;
  const uint32_t blk = ld32(rs, 64u + 4u * (uint32_t)prow) + before;
  uint32_t bad = ((uint64_t)blk + total > ch.W) ? 1u : 0u;
  const uint32_t blk_byte = ch.off_pay + 4u * blk;
  Words wd;
  wd.m = m;
  wd.us = 16u * ns;
  wd.a0 = blk_byte + 16u * (uint32_t)lane;
  wd.t0 = blk_byte + 4u * (4u * m * ns + incl - tl) - 16u * m;

  // ring word k (stream word k, complemented) in slot k mod 16
  auto put = [&](uint32_t k, uint32_t w) { ring[((k % kAncRing) << 6) + lane] = ~w; };
  auto get = [&](uint32_t k) { return ring[((k % kAncRing) << 6) + lane]; };
  auto put_unit = [&](uint32_t k, const u32x4& u) {
    put(k, u.x);
    put(k + 1, u.y);
    put(k + 2, u.z);
    put(k + 3, u.w);
  };
  {
    const u32x4 u0 = Block<4>::load(rs, wd.unit(0)).v, u1 = Block<4>::load(rs, wd.unit(1)).v;
    put_unit(0, u0);
    put_unit(4, u1);
  }
  uint32_t landed = 8;  // ring words landed
  u32x4 pend = Block<4>::load(rs, wd.unit(2)).v;
  bool inflight = true;
  uint32_t ncode = get(0), range = 0xFFFFFFFFu;
  uint32_t p = 32;  // stream bits shifted into the code
  // the bisection's first two levels are the same keys for every lane:
  // cum[128], then cum[64] or cum[192]
  const uint32_t key128 = cum[128], key64 = cum[64], key192 = cum[192];

  // one symbol whose next stream bits are x (complemented); returns s and
  // leaves the shift and its selector in sh, sel
  constexpr uint32_t cum0 = 0;  // LDS byte address of cum[0]
  auto symbol = [&](uint32_t x, uint32_t& sh, uint32_t& sel) -> uint32_t {
    const uint32_t r = range >> kProbBits;
    // ad = byte offset 4 s of the symbol being bisected
    const uint32_t m1 = le_mask(r, key128, ncode);
    uint32_t ad = m1 & (128u * 4u);
    ad |= le_mask(r, bit_select(m1, key192, key64), ncode) & (64u * 4u);
#pragma unroll
    for (uint32_t stp = 32; stp; stp >>= 1) ad |= le_mask(r, lds32(cum0 + ad + 4u * stp), ncode) & (4u * stp);
    const uint32_t c0 = lds32(cum0 + ad), c1 = lds32(cum0 + ad + 4u);
    const uint32_t sym = ad >> 2;
    ncode += mul24(r, c0);  // code -= r * cum[s]
    const uint32_t rn = mul24(r, c1 - c0);
    sh = (uint32_t)__builtin_clz(rn) & 24u;
    range = rn << sh;
    sel = shift_sel(sh);
    ncode = __builtin_amdgcn_perm(ncode, x, sel);
    return sym;
  };
  // this (kv, layer)'s anchors [ng][C] through a buffer resource: the channel is
  // the vector offset, the group's row a wave-uniform scalar offset
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ch.out + (size_t)arow * ch.ng * a.C), 0, (int)((uint32_t)ch.ng * (uint32_t)a.C),
      kBufRsrcWord3);
  auto put_anchor = [&](int g, uint32_t sym) {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(sym ^ 0x80u), ro, (uint32_t)c,
                                         (uint32_t)g * (uint32_t)a.C, 0);
  };
  // n (1 or 2) symbols from the 64-bit window at bit p
  auto pair = [&](int g, int n) {
    const uint32_t j = p >> 5, o = p & 31u;
    const uint32_t w0 = get(j), w1 = get(j + 1), w2 = get(j + 2);
    const uint32_t hi = (uint32_t)((((uint64_t)w0 << 32) | w1) << o >> 32);
    const uint32_t lo = (uint32_t)((((uint64_t)w1 << 32) | w2) << o >> 32);
    uint32_t sh1, sel1, sh2, sel2;
    put_anchor(g, symbol(hi, sh1, sel1));  // anchor s - 128: s with its top bit flipped
    p += sh1;
    if (n == 2) {
      put_anchor(g + 1, symbol(__builtin_amdgcn_perm(hi, lo, sel1), sh2, sel2));
      p += sh2;
    }
  };
  auto ring_step = [&]() {
    if (inflight) {
      put_unit(landed, pend);
      landed += 4;
    }
    // the next unit lands over ring words already consumed (lanes without
    // room point their load past the blob end: no memory access)
    inflight = landed + 4u - (p >> 5) <= kAncRing;
    pend = Block<4>::load(rs, inflight ? wd.unit(landed >> 2) : 0xFFFFFFF0u).v;
  };
  int g = 0;
  for (; g + kAncRound <= ch.ng; g += kAncRound) {
#pragma unroll
    for (int i = 0; i < kAncRound; i += 2) pair(g + i, 2);
    ring_step();
  }
  for (; g + 1 < ch.ng; g += 2) pair(g, 2);  // the last round needs no more words
  if (g < ch.ng) pair(g, 1);
  // a valid stream keeps code < range throughout; a corrupt one breaks it for good
  bad |= (~ncode >= range) ? 1u : 0u;
  if (bad) atomicOr(a.status, 1u);
}

}  // namespace

namespace {
template <bool PG>
void launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)(a.n_groups * a.L * a.nblk);
  const dim3 grid(blocks), block(2 * kLanes * a.waves + (a.warm_wave ? kLanes : 0));
  if (a.waves == 1) {  // one chunk per workgroup: small rings, eight workgroups per CU
    const size_t lds = reg_ring_base() + (size_t)2 * reg_ring_bytes();
    if (a.G == 10)
      k_decode_reg<10, PG><<<grid, block, lds, st>>>(a);
    else
      k_decode_reg<0, PG><<<grid, block, lds, st>>>(a);
  } else {
    const size_t lds = kTabBytes + (size_t)2 * a.waves * win_ring_bytes();
    if (a.G == 10)
      k_decode_win<10, PG><<<grid, block, lds, st>>>(a);
    else
      k_decode_win<0, PG><<<grid, block, lds, st>>>(a);
  }
}
}  // namespace

hipError_t launch_anchor_decode(const AnchorDecodeArgs& a, hipStream_t st) {
  if (a.nchunks > 0)
    k_anchor_decode<<<dim3((unsigned)((a.nblk + kAncWaves - 1) / kAncWaves), (unsigned)(2 * a.L),
                           (unsigned)a.nchunks),
                      64 * kAncWaves, kAncLds, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.paged)
    launch_decode_t<true>(a, st);
  else
    launch_decode_t<false>(a, st);
  return hipGetLastError();
}

}  // namespace cg
