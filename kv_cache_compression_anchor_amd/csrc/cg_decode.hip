// Chunk decoder (gptget 方法详解: the receiver decodes the bitstream on the GPU;
// CacheGen blog, section 2.1: anchor plus delta reconstruction).
//
// One lane per stream (kv, layer, channel), one wave per (chunk, kv), one
// workgroup per (group of chunks with the same quality, layer, 64-channel
// block): the workgroup stages the block's 2 x 64 cumulative tables (K and V)
// in LDS once and every wave decodes its chunk's K or V streams against them.  All lanes of a wave sit on the same token,
// so each reconstructed token row is one coalesced 128-byte store.  Blob bytes
// are read through a buffer resource bounded by the blob size: a corrupt blob
// reads zeros past its end instead of faulting.
#include "cg_internal.h"

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

// The kernel's LDS is all dynamic, so it starts at LDS address 0: pointers are
// formed from byte addresses directly (constant parts of an address then fold
// into the instructions' offset fields).
template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_at(uint32_t byte_addr) {
  return reinterpret_cast<__attribute__((address_space(3))) T*>(static_cast<uintptr_t>(byte_addr));
}

__device__ __forceinline__ uint32_t lds32(uint32_t addr) { return *lds_at<uint32_t>(addr); }
__device__ __forceinline__ uint32_t lds16(uint32_t addr) { return *lds_at<uint16_t>(addr); }

// a block's words into consecutive ring slots (slots are 256 bytes apart)
__device__ __forceinline__ void lds_put(uint32_t lane_addr, uint32_t slot_off, const Block<2>& b) {
  auto p = lds_at<uint32_t>(lane_addr + slot_off);
  p[0] = b.v.x;
  p[64] = b.v.y;
}
__device__ __forceinline__ void lds_put(uint32_t lane_addr, uint32_t slot_off, const Block<4>& b) {
  auto p = lds_at<uint32_t>(lane_addr + slot_off);
  p[0] = b.v.x;
  p[64] = b.v.y;
  p[128] = b.v.z;
  p[192] = b.v.w;
}

// (float)((x >> 8) & 0xFF) in one instruction
__device__ __forceinline__ float byte1_to_float(uint32_t x) {
  float f;
  asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(x));
  return f;
}

// The workgroup's LDS holds the K and V tables of one (layer, 64-channel block)
// side by side: row k = [cum[k] of the 64 K streams | cum[k] of the 64 V
// streams], 256 bytes, so the byte address of entry k of a lane is
// k * 256 + (kv * 128 + 2 * slot) and bits 8..15 of it are k itself.
constexpr uint32_t kRow = 4 * kLanes;
constexpr uint32_t kTabBytes = kImgRows * kRow;        // 16,640
// A wave's word ring: 2 * RB slots (two blocks of RB words) x 64 lanes x 4 B.
// The first wave's ring is aligned to the ring size, so a slot address is the
// lane's ring address with the slot number in the bits above 7.
__host__ __device__ constexpr uint32_t ring_bytes(int rb) { return 2u * rb * 4u * kLanes; }
__host__ __device__ constexpr uint32_t ring_base(int rb) {
  return (kTabBytes + ring_bytes(rb) - 1) / ring_bytes(rb) * ring_bytes(rb);
}

// All ones when r * key <= code, else zero.  ncode is ~code, so the 64-bit sum
// r * key + (2^64 - code - 1) stays within [2^64 - 2^32, 2^64) when
// r * key <= code and otherwise wraps to r * key - code - 1 < 2^32: its high
// word is the mask (one v_mad_u64_u32; r * key < 2^32).
__device__ __forceinline__ uint32_t le_mask(uint32_t r, uint32_t key, uint32_t ncode) {
  const uint64_t c = 0xFFFFFFFF00000000ull | ncode;
  return (uint32_t)(((uint64_t)r * key + c) >> 32);
}

// GS: group size fixed at compile time (0 = the runtime a.G only).
// RB: words per fetched block (4 in workgroups of several chunks; 2 when a
// workgroup holds one chunk, so that eight of them fit a CU's LDS).
template <int GS, int RB>
__global__ __launch_bounds__(512) void k_decode(DecodeArgs a) {
  // LDS: the tables at 0 ([65 rows][K: 64 u16 | V: 64 u16]), then one word
  // ring per wave ([2 RB slots][64 lanes] u32)
  auto tab = lds_at<uint32_t>(0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int kv = wave & 1;
  const int ci = a.groups[grp].chunk[wave >> 1];
  if (ci < 0) return;
  const DecChunk ch = a.chunks[ci];
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)ch.blob, 0, (int)ch.blob_bytes, kBufRsrcWord3);
  const int row = kv * a.L + l;

  const int c = cb * kLanes + lane;
  const bool active = c < a.C;

  // start of this lane's stream: row offset + lengths of the streams before it
  // (the whole wave takes part in the prefix sums)
  const uint32_t len_base = ch.off_len + 2u * (uint32_t)row * (uint32_t)a.C;
  uint32_t before = 0;
  for (int j = lane; j < cb * kLanes; j += kLanes) before += ld16(rs, len_base + 2u * j);
  for (int o = 32; o; o >>= 1) before += __shfl_xor(before, o);
  const uint32_t my_len = active ? ld16(rs, len_base + 2u * c) : 0u;
  uint32_t incl = my_len;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (!active) return;  // no cross-lane work below
  const uint32_t start = ld32(rs, 64u + 4u * row) + before + incl - my_len;
  uint32_t bad = ((uint64_t)start + my_len > ch.W) ? 1u : 0u;

  const size_t pi = (size_t)row * a.C + c;
  const float scale_a = a.scale_a[pi];
  const float step = a.step[q][pi];

  const uint32_t lane_addr = (uint32_t)kv * (2u * kLanes) + 2u * lane_slot(lane);
  const uint32_t key32 = lds16(lane_addr + 32u * kRow);  // root of the search

  // decoder state: ncode = ~code; range; bb = the next bits of the stream,
  // complemented, in its low `left` bits (most significant first, 32..64 of
  // them before every pair of symbols).  Words 0..2 start the state; words 3..
  // reach bb through the wave's LDS ring: word 3 + i sits in slot i mod 2 RB of
  // the lane's column, fetched RB words at a time one group ahead of use.
  const uint32_t sbase = ch.off_pay + 4u * start;  // byte offset of word 0
  uint32_t ncode = ~ld32(rs, sbase);
  uint64_t bb = ((uint64_t)~ld32(rs, sbase + 4u) << 32) | ~ld32(rs, sbase + 8u);
  uint32_t left = 64;
  uint32_t range = 0xFFFFFFFFu;
  constexpr uint32_t kSlotMask = (2u * RB - 1u) << 8;
  const uint32_t ring = ring_base(RB) + (uint32_t)wave * ring_bytes(RB) + 4u * (uint32_t)lane;
  // ring words taken and written, counted in units of 256 (one slot's size)
  uint32_t taken = 0;
  uint32_t landed = (2u * RB) << 8;                  // words 3 .. 2 RB + 2, written below
  uint32_t fetch_off = sbase + 12u + 8u * RB;        // the next block
  {
    const Block<RB> b0 = Block<RB>::load(rs, sbase + 12u);
    const Block<RB> b1 = Block<RB>::load(rs, sbase + 12u + 4u * RB);
    lds_put(ring, 0u, b0);
    lds_put(ring, (uint32_t)RB << 8, b1);
  }
  Block<RB> pend = {};  // block in flight
  bool inflight = false;

  // output rows of this (kv, layer, chunk) through a buffer resource: the lane's
  // channel is the vector offset, the token row a wave-uniform scalar offset
  uint16_t* const out_base = (kv ? a.v_out : a.k_out) + ((size_t)l * a.T + ch.t0) * a.C;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      out_base, 0, (int)((uint32_t)ch.tc * (uint32_t)a.C * 2u), kBufRsrcWord3);
  const uint32_t row_bytes = 2u * (uint32_t)a.C;
  const uint32_t lane_off = 2u * (uint32_t)c;
  const uint32_t anc_base = ch.off_anchor + (uint32_t)row * (uint32_t)ch.ng * (uint32_t)a.C + c;
  int anc_next = ld8s(rs, anc_base);

  // one symbol: search, interval update, renormalisation, reconstruction
  auto symbol = [&](uint32_t soff, float base) {
    const uint32_t r = range >> kProbBits;
    // largest s with r * cum[s] <= code, as the LDS address of cum[s]
    uint32_t ad = lane_addr | (le_mask(r, key32, ncode) & (32u * kRow));
#pragma unroll
    for (uint32_t stp = 16; stp; stp >>= 1) ad |= le_mask(r, lds16(ad + stp * kRow), ncode) & (stp * kRow);
    const uint32_t c0 = lds16(ad), c1 = lds16(ad + kRow);
    ncode += mul24(r, c0);  // code -= r * cum[s]
    const uint32_t rn = mul24(r, c1 - c0);
    // shift in whole bytes until range >= 2^24 (0, 1 or 2 bytes; rn >= 2^9)
    const uint32_t sh = (uint32_t)__builtin_clz(rn) & 24u;
    range = rn << sh;
    const uint32_t t = left - sh;
    ncode = (ncode << sh) | __builtin_amdgcn_ubfe((uint32_t)(bb >> (t & 63u)), 0u, sh);
    left = t;
    const float y = __builtin_fmaf(byte1_to_float(ad), step, base);
    __builtin_amdgcn_raw_buffer_store_b16(float_to_half_bits(y), ro, lane_off, soff, kStoreNT);
  };

  // A lane takes a word when fewer than 32 bits remain (two symbols need at
  // most 32).  Only stores go to memory inside a group, so no wait in it
  // drains them; a ring that has run dry (more than the buffered words taken
  // in one group, which typical data never does) falls back to a direct load.
  auto refill = [&]() {
    const bool take = left < 32;
    const uint32_t slot = (taken & kSlotMask) | ring;
    if (take && taken >= landed)
      *lds_at<uint32_t>(slot) = ld32(rs, sbase + 12u + (taken >> 6));
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
      lds_put(ring, landed & ((uint32_t)RB << 8), pend);
      landed += (uint32_t)RB << 8;
    }
    inflight = landed + ((uint32_t)RB << 8) <= taken + ((2u * RB) << 8);
    pend = Block<RB>::load(rs, inflight ? fetch_off : 0xFFFFFFF0u);
    if (inflight) fetch_off += 4u * RB;
  };

  // one group: the anchor row, then its deltas in pairs (a lone last one when
  // the group has an even number of tokens)
  auto group = [&](int g, int ta, int te) {
    ring_step();
    const int anc = anc_next;
    anc_next = ld8s(rs, anc_base + (uint32_t)(g + 1) * a.C);  // past the last group: unused
    const float ahat = anchor_value(anc, scale_a);
    __builtin_amdgcn_raw_buffer_store_b16(float_to_half_bits(ahat), ro, lane_off,
                                          (uint32_t)ta * row_bytes, kStoreNT);
    const float base = __builtin_fmaf(-32.0f, step, ahat);
    int t = ta + 1;
#pragma unroll
    for (; t + 1 < te; t += 2) {
      // keep the refill after the previous pair's stores: its wait then
      // leaves those two stores in flight
      __builtin_amdgcn_sched_barrier(0);
      refill();
      symbol((uint32_t)t * row_bytes, base);
      symbol((uint32_t)(t + 1) * row_bytes, base);
    }
    if (t < te) {
      __builtin_amdgcn_sched_barrier(0);
      refill();
      symbol((uint32_t)t * row_bytes, base);
    }
  };

  // everything loaded so far (scale, step, first words, first anchor) is in
  // registers before the loop, so no wait inside it is for those loads
  __builtin_amdgcn_s_waitcnt(0);
  int g = 0;
  if constexpr (GS > 0) {
    // full groups of the compile-time size: the same loads and stores every
    // iteration, so the anchor loaded one group ahead is waited for without
    // waiting for the stores issued since
    const int nfull = ch.tc / GS;
    for (; g < nfull; g++) group(g, g * GS, g * GS + GS);
  }
  for (; g < ch.ng; g++) group(g, g * a.G, min(g * a.G + a.G, ch.tc));
  // a valid stream keeps code < range throughout; a corrupt one breaks it for good
  bad |= (~ncode >= range) ? 1u : 0u;
  if (bad) atomicOr(a.status, 1u);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)(a.n_groups * a.L * a.nblk);
  const dim3 grid(blocks), block(2 * kLanes * a.waves);
  if (a.waves == 1) {  // one chunk per workgroup: small rings
    const size_t lds = ring_base(2) + (size_t)2 * a.waves * ring_bytes(2);
    if (a.G == 10)
      k_decode<10, 2><<<grid, block, lds, st>>>(a);
    else
      k_decode<0, 2><<<grid, block, lds, st>>>(a);
  } else {
    const size_t lds = ring_base(4) + (size_t)2 * a.waves * ring_bytes(4);
    if (a.G == 10)
      k_decode<10, 4><<<grid, block, lds, st>>>(a);
    else
      k_decode<0, 4><<<grid, block, lds, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace cg
