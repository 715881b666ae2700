// Chunk encoder (CacheGen blog, section 2.1: anchor quantised to 8 bits, deltas
// of the other tokens of the group against it, layer-group step, arithmetic
// coding).  One lane per stream (kv, layer, channel): a wave codes 64 channels
// of one (kv, layer) row in lockstep, so every input row it reads is one
// coalesced 128-byte segment.  Streams land in per-stream scratch, 16 bytes at
// a time, then a wavefront prefix sum over the stream lengths packs them into
// the blob.
#include "cg_build.h"

namespace cg {
namespace {

// Range coder of one lane, producing the same bytes as a byte-at-a-time coder
// with carry propagation, a whole 32-bit word at a time: `L` holds the coder's
// 32-bit low window plus up to three output bytes not yet taken above it, so a
// carry out of the window simply runs into those bytes.  A word leaves `L` once
// four bytes sit above the window; the last one taken (`W`) and a run of
// 0xFFFFFFFF words after it (`P`) stay open until no carry can reach them.
// `W` always has a slot: before the first word is taken it is a placeholder
// word in front of the stream, which the first emission fills and nothing reads
// (no carry can reach past the first word; it stays in the staging ring below
// and is never written out).
struct RcEnc {
  uint64_t L;      // window (bits 0..31) and the bytes above it (bits 32..32+kh-1)
  uint32_t kh;     // 8 * bytes above the window: 0..24; plus 64 while P != 0
  uint32_t range;
  uint32_t W;      // last word taken out of L, not final yet
  uint32_t P;      // 0xFFFFFFFF words after W, not final yet
  uint32_t Y;      // 0 while P != 0, else 0xFFFFFFFF
};

// A lane's output words go to a staging ring in LDS of RW = 4 or 8 words per
// lane ([slot][64 lanes], RW x 256 bytes per wave and aligned to that, so slot
// k of the lane is at base | 256 k and the lanes' words of one emission are
// conflict-free), and each completed 16-byte unit (words 4u .. 4u + 3) is
// written to the wave's scratch block, laid out [unit][64 lanes][4 words], with
// one store: a quarter of the stores of writing words one by one, each lane's
// 16 bytes in one cache line where single words of 64 lanes at different
// positions touched up to 64 lines per store.  Word w of the stream is
// emission w + 1 (emission 0 is the placeholder W starts as, which lands in
// the ring's last slot and is never written out).
constexpr uint32_t kUnitRowBytes = 16u * kLanes;  // one unit of each of the 64 streams
template <int RW>
struct Sink {
  static_assert(RW == 4 || RW == 8, "a ring of one or two units");
  static constexpr uint32_t smask = 256u * (RW - 1);     // the slot bits of sa
  static constexpr uint32_t umask = 1024u * (RW / 4 - 1);  // the bit of uoff that is the unit's half of the ring
  __amdgpu_buffer_rsrc_t rs;  // the wave's scratch block
  uint32_t base;   // LDS byte address of the lane's slot 0
  uint32_t sa;     // 256 (emissions + 7): the next slot is (sa >> 8) mod RW
  uint32_t fnext;  // sa once the next unit to write out is complete: 256 (12 + 4 u)
  uint32_t uoff;   // scratch byte offset of that unit: 1024 u + 16 lane
};

template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_ptr(uint32_t byte_addr) {
  return reinterpret_cast<__attribute__((address_space(3))) T*>(static_cast<uintptr_t>(byte_addr));
}

// the next word into the ring
template <class S>
__device__ __forceinline__ void stage_word(S& o, uint32_t w) {
  *lds_ptr<uint32_t>(o.base | (o.sa & S::smask)) = w;
  asm("v_add_u32 %0, 0x100, %0" : "+v"(o.sa));  // in place, after the address is formed
}

// writes the unit at fnext out of the ring (with 8 slots, slot bit 2 of its
// words is u & 1, which is bit 10 of uoff)
template <class S>
__device__ __forceinline__ void write_unit(S& o) {
  const uint32_t a = o.base | (o.uoff & S::umask);
  const uint32_t w0 = *lds_ptr<uint32_t>(a), w1 = *lds_ptr<uint32_t>(a + 256u);
  const uint32_t w2 = *lds_ptr<uint32_t>(a + 512u), w3 = *lds_ptr<uint32_t>(a + 768u);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = {w0, w1, w2, w3};
  __builtin_amdgcn_raw_buffer_store_b128(v, o.rs, o.uoff, 0, 0);
  o.uoff += kUnitRowBytes;
  o.fnext += 1024u;
}

// the lanes whose next unit is complete write it out (at most one: callers
// flush before more than RW - 3 words have been staged since the last flush)
template <class S>
__device__ __forceinline__ void flush_units(S& o) {
  if (o.sa >= o.fnext) write_unit(o);
}

// one word of the general steps: staged and, once its unit is complete,
// written out at once (they may take several words in one symbol)
template <class S>
__device__ __forceinline__ void emit_word(S& o, uint32_t w) {
  stage_word(o, w);
  flush_units(o);
}

// the last, partial unit (its other slots hold stale words, which nothing reads)
template <class S>
__device__ __forceinline__ void flush_tail(S& o) {
  if (o.sa > o.fnext - 1024u) write_unit(o);
}

// words of the stream taken so far
template <class S>
__device__ __forceinline__ uint32_t sink_words(const S& o) {
  return o.sa >= 2048u ? (o.sa >> 8) - 8u : 0u;
}

// a lane's sink over the wave's scratch block (swb words per stream) and its
// column of the wave's ring (LDS byte address ring, RW x 256 aligned)
template <int RW>
__device__ __forceinline__ Sink<RW> make_sink(uint32_t* block, size_t swb, uint32_t ring, int lane) {
  Sink<RW> o;
  o.rs = __builtin_amdgcn_make_buffer_rsrc(block, 0, (int)(4u * kLanes * (uint32_t)swb), kBufRsrcWord3);
  o.base = ring + 4u * (uint32_t)lane;
  o.sa = 7u * 256u;
  o.fnext = 12u * 256u;
  o.uoff = 16u * (uint32_t)lane;
  return o;
}

// LDS of the encode kernels, all dynamic so that it starts at address 0: the
// waves' rings first (each aligned to its size), then the kernel's table
extern __shared__ __attribute__((aligned(16))) uint8_t enc_lds[];

// --- general steps: every case, used for the rare symbols and the flush ----

// a carry reached an all-ones run: it wraps to zeros, W + 1 and all but the
// last zero word are final, the last zero word stays open
template <class S>
__device__ __forceinline__ void carry_into_run(RcEnc& e, S& o) {
  emit_word(o, e.W + 1u);
  for (uint32_t j = 1; j < e.P; j++) emit_word(o, 0u);
  e.W = 0;
  e.P = 0;
}

// the carry out of the held bytes after an addition to L: into W, or through
// an all-ones run
template <class S>
__device__ __forceinline__ void settle_carry(RcEnc& e, S& o) {
  const uint32_t hmask = (1u << e.kh) - 1u;
  uint32_t hi = (uint32_t)(e.L >> 32);
  const bool c = hi > hmask;
  hi &= hmask;
  e.L = ((uint64_t)hi << 32) | (uint32_t)e.L;
  if (c && e.P) {
    carry_into_run(e, o);
  } else {
    e.W += c ? 1u : 0u;
  }
}

// shift nb8 / 8 (0..2) bytes out of the window; a word leaves when four are
// held after the shift: it is the four top bytes of L before it
template <class S>
__device__ __forceinline__ void shift_bytes(RcEnc& e, uint32_t nb8, S& o) {
  const uint32_t lo = (uint32_t)e.L, hi = (uint32_t)(e.L >> 32);
  const uint32_t kh2 = e.kh + nb8;
  const bool ext = kh2 >= 32u;
  const uint32_t wn = __builtin_amdgcn_alignbit(hi, lo, e.kh);
  const uint32_t lo_k = ext ? __builtin_amdgcn_ubfe(lo, 0u, e.kh) : lo;
  const uint32_t hi_k = ext ? 0u : hi;
  e.L = (((uint64_t)hi_k << 32) | lo_k) << nb8;
  e.kh = kh2 & 31u;
  if (ext) {
    if (wn == 0xFFFFFFFFu) {
      e.P++;  // may still wrap
    } else {
      emit_word(o, e.W);
      for (; e.P; e.P--) emit_word(o, 0xFFFFFFFFu);
      e.W = wn;
    }
  }
}

// --- one symbol -----------------------------------------------------------
// The common case (no all-ones run open, and no all-ones word taken) runs
// branch-free for the whole wave; a lane in a rare case redoes the symbol from
// its previous state with the general steps, in a branch the wave takes only
// when some lane needs it.  A lane with a run open always takes that branch:
// its kh carries bit 6, so kh + nb8 >= 32 (shifts and bit-field widths read
// only the low five bits of kh), and its Y is 0, so wn >= Y; then "a word
// leaves and it is all ones, or a run is open" is one compare pair.
template <class S>
__device__ __forceinline__ void rc_put(RcEnc& e, uint32_t c0, uint32_t freq, S& o) {
  const RcEnc e0 = e;
  const uint32_t r = e.range >> kProbBits;
  const uint64_t L1 = e.L + (uint64_t)r * c0;  // one 32 x 32 -> 64 multiply-add
  const uint32_t lo = (uint32_t)L1, hx = (uint32_t)(L1 >> 32);
  // the held bytes are below 2^kh and r c0 below 2^32, so the carry out of
  // them is bit kh of hx, and nothing above it
  const uint32_t cy = hx >> (e.kh & 31u);
  const uint32_t rn = mul24(r, freq);
  const uint32_t nb8 = (uint32_t)__builtin_clz(rn) & 24u;  // renormalise while range < 2^24
  const uint32_t kh2 = e.kh + nb8;
  // the four top bytes of the window and held bytes (the carry bit lies above)
  const uint32_t wn = __builtin_amdgcn_alignbit(hx, lo, e.kh);
  // lane masks of "a word leaves" and "it is all ones or a run is open": the
  // rare lanes are both, the emitting lanes the first only (as masks, so that
  // each compare is made once)
  const uint64_t m_ext = __builtin_amdgcn_ballot_w64(kh2 >= 32u);
  const uint64_t m_ge = __builtin_amdgcn_ballot_w64(wn >= e.Y);
  const bool rare = __builtin_amdgcn_inverse_ballot_w64(m_ext & m_ge);
  const uint32_t W1 = e.W + cy;
  const bool emit = __builtin_amdgcn_inverse_ballot_w64(m_ext & ~m_ge);
  if (emit) stage_word(o, W1);
  e.W = emit ? wn : W1;
  // shifted by nb8, L keeps its low 32 + (kh2 mod 32) bits: without a word
  // leaving that is all of it less the carry; with one, the window's low kh
  // bits, moved up
  const uint64_t Ls = L1 << nb8;
  e.kh = kh2 & 95u;  // mod 32, keeping bit 6 (an open run's lanes take the branch below)
  e.L = ((uint64_t)__builtin_amdgcn_ubfe((uint32_t)(Ls >> 32), 0u, e.kh) << 32) | (uint32_t)Ls;
  e.range = rn << nb8;
  if (rare) {
    RcEnc s = e0;
    s.kh &= 31u;
    s.L = L1;
    settle_carry(s, o);
    s.range = rn << nb8;
    shift_bytes(s, nb8, o);
    e = s;
    e.kh |= s.P != 0u ? 64u : 0u;
    e.Y = s.P != 0u ? 0u : 0xFFFFFFFFu;
  }
}

// Flush: the fewest bytes (one or two) that name an aligned block inside
// [low, low + range), so the stream decodes whatever bytes follow it; then the
// open words and the bytes still held, the last word padded with zero bytes.
template <class S>
__device__ __forceinline__ void rc_finish(RcEnc& e, S& o) {
  e.kh &= 31u;
  const uint64_t win = e.L & 0xFFFFFFFFull;
  uint32_t nb8 = 8;
  uint64_t V = (win + 0xFFFFFFull) & ~0xFFFFFFull;
  if (V + 0x1000000ull > win + e.range) {
    nb8 = 16;
    V = (win + 0xFFFFull) & ~0xFFFFull;
  }
  e.L = e.L - win + V;
  settle_carry(e, o);
  shift_bytes(e, nb8, o);
  emit_word(o, e.W);  // the placeholder when no word was taken
  for (; e.P; e.P--) emit_word(o, 0xFFFFFFFFu);
  const uint32_t k = e.kh >> 3;
  if (k) emit_word(o, (uint32_t)(e.L >> 32) << (8u * (4u - k)));
}

// A workgroup is (group of up to 4 blobs of one quality, kv, layer, 64-channel
// block) with one wave per blob: the block's cumulative table is staged in LDS
// once for all of them.  A launch covers up to kEncMaxBlobs (chunk, quality)
// blobs of the same tensors so that enough waves are in flight to hide the
// latency of each lane's serial coder.
constexpr int kEncMaxWaves = 4;

// K/V are read once per blob and streamed: non-temporal loads, so that they
// do not push out of the L2 the scratch lines that the wave's lanes are still
// filling one word at a time (evicted half-written, a line is written to memory
// again for every part: 8% of the encode time on the Mistral-7B shape)
constexpr int kLoadNT = 2;

__device__ __forceinline__ uint32_t ld_half(__amdgpu_buffer_rsrc_t r, uint32_t lane_off,
                                            uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, lane_off, soff, kLoadNT);
}

// GS: group size fixed at compile time (0 = the runtime a.G only).  With GS,
// the input of full groups is loaded two groups ahead, so the wait for it
// never includes the stores issued since (every group issues the same loads).
// RW: ring words per lane (8 where the launch's workgroups fit a compute unit
// with them, else 4); the ring of RW words holds RW - 3 staged words beyond a
// partial unit, so the delta loop flushes every 3 symbols with 8 and every
// symbol with 4.
template <int GS, int RW>
__global__ __launch_bounds__(kLanes * kEncMaxWaves) void k_encode(EncodeArgs a) {
  uint16_t* tab = reinterpret_cast<uint16_t*>(enc_lds + (size_t)a.waves * RW * 256u);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int per_grp = a.nrows * a.nblk;
  const int grp = blockIdx.x / per_grp, unit = blockIdx.x % per_grp;
  // The workgroups that share a compute unit are ncu apart in launch order,
  // and a stream's cost grows with its bits per symbol: finer steps (shallow
  // layers) and outlier channels cost more.  So that each compute unit gets a
  // mix, the second half of the launch's rows is taken in reverse order (the
  // V rows of a whole-row launch: deep layers beside the K rows' shallow ones)
  // and the blocks of a row are rotated by 5 per ncu workgroups (neighbouring
  // rows on one compute unit take different channel blocks).  The map is one
  // to one on the units of the launch.
  const int prow = unit / a.nblk, pcb = unit % a.nblk;
  const int half = a.nrows >> 1;
  const int rrel = prow >= half ? half + (a.nrows - 1 - prow) : prow;  // row within the launch's range
  const int row = a.row0 + rrel;  // kv * L + l
  const int cb = (pcb + 5 * ((prow * a.nblk) / a.ncu)) % a.nblk;
  // (the group's blob indices read from the arguments, not copied to a local
  // array: indexing that by wave would take it through private memory)
  const EncGroup& eg = a.groups[grp];
  {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(
        a.b[eg.blob[0]].img + ((size_t)row * a.nblk + cb) * kImgRows * kLanes);
    uint32_t* dst = reinterpret_cast<uint32_t*>(tab);
    for (int j = threadIdx.x; j < kImgRows * kLanes / 2; j += blockDim.x) dst[j] = src[j];
  }
  __syncthreads();
  // wave-uniform, so that the blob's fields and buffer resources live in SGPRs
  const int bi = __builtin_amdgcn_readfirstlane(eg.blob[wave]);
  if (bi < 0) return;
  const EncBlob& B = a.b[bi];
  const int kv = row / a.L;
  const int l = row % a.L;
  const int c = cb * kLanes + lane;
  if (c >= a.C) return;
  const size_t pi = ((size_t)kv * a.L + l) * a.C + c;
  const float scale_a = a.scale_a[pi], inv_a = a.inv_a[pi], inv_step = B.inv_step[pi];
  // the chunk's rows of this (kv, layer): the lane's channel is the vector
  // offset, the token row a scalar offset.  The scalar offset is outside the
  // buffer's range check, so no load may name a row at or past tc.
  const uint32_t row_bytes = 2u * (uint32_t)a.C;
  const __amdgpu_buffer_rsrc_t xin = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((kv ? a.v : a.k) + ((size_t)l * a.T + B.t0) * a.C), 0,
      (int)((uint32_t)B.tc * row_bytes), kBufRsrcWord3);
  const uint32_t lane_off = 2u * (uint32_t)c;
  // the wave's block of 64 streams in scratch, swb words each, as 16-byte units
  const size_t block = (size_t)rrel * a.nblk + cb;
  Sink<RW> o = make_sink<RW>(B.scratch + block * kLanes * a.swb, a.swb, (uint32_t)wave * RW * 256u, lane);
  // raw anchors into the blob, [ng][C] for this (kv, layer): the lane's
  // channel is the vector offset, the group a scalar offset; coded anchors are
  // coded from the input by k_anchor_encode instead (a wave-uniform choice)
  const bool raw_anchors = B.lay.off_anchor != 0;
  const __amdgpu_buffer_rsrc_t anc = __builtin_amdgcn_make_buffer_rsrc(
      B.blob + B.lay.off_anchor + ((size_t)kv * a.L + l) * B.ng * a.C, 0,
      (int)((uint32_t)B.ng * (uint32_t)a.C), kBufRsrcWord3);
  RcEnc e = {0, 0u, 0xFFFFFFFFu, 0u, 0u, 0xFFFFFFFFu};
  // sum of 0 x every input: zero unless some input is infinite or NaN
  float nfacc = 0.0f;

  // a delta's table row as a byte offset: (level + 32) * 128 + the lane's
  // column, level + 32 = level_bits(u) - (kLevelBias - 32)
  const uint32_t row0 = (uint32_t)(2 * lane_slot(lane)) - ((uint32_t)(kLevelBias - 32) << 7);
  const uint8_t* tab8 = reinterpret_cast<const uint8_t*>(tab);

  // one group from its tokens' binary16 bits: the anchor, then the deltas
  auto code_group = [&](int g, int n, auto half_of) {
    const float x0 = half_bits_to_float(half_of(0));
    nfacc = __builtin_fmaf(x0, 0.0f, nfacc);
    const int32_t ab = anchor_bits(x0, inv_a);
    if (raw_anchors)
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)ab, anc, (uint32_t)c, (uint32_t)g * (uint32_t)a.C, 0);
    const float ahat = anchor_of_bits(ab) * scale_a;  // anchor_value of the code
    for (int j = 1; j < n; j++) {
      const float xf = half_bits_to_float(half_of(j));
      nfacc = __builtin_fmaf(xf, 0.0f, nfacc);
      const uint32_t off = ((uint32_t)level_bits((xf - ahat) * inv_step) << 7) + row0;
      const uint32_t c0 = *reinterpret_cast<const uint16_t*>(tab8 + off);
      const uint32_t c1 = *reinterpret_cast<const uint16_t*>(tab8 + off + 2 * kLanes);
      rc_put(e, c0, c1 - c0, o);
      // the common step stages at most one word
      if (RW == 4 || j % 3 == 0 || j == n - 1) flush_units(o);
    }
  };

  int g = 0;
  const int nfull = GS > 0 ? B.tc / GS : 0;
  if (GS > 0 && nfull > 0) {
    constexpr int NG = GS > 0 ? GS : 1;
    uint32_t xa[NG], xb[NG];
    // A prefetch of a group past the last full one is never coded (the loop
    // below ends first); it re-reads the last full group instead, so every
    // row read lies inside the chunk.
    auto load = [&](uint32_t (&xv)[NG], int gg) {
      const int gl = min(gg, nfull - 1);
#pragma unroll
      for (int j = 0; j < NG; j++) xv[j] = ld_half(xin, lane_off, (uint32_t)(gl * NG + j) * row_bytes);
    };
    load(xa, 0);
    load(xb, 1);
    // In a launch whose waves are all resident at once, waves that have done
    // less run first: a SIMD issues from its oldest ready wave, so otherwise
    // the last-dispatched waves run last with few waves left beside them.
    // Each wave steps its priority down at half, three quarters and seven
    // eighths of its pairs of groups.  (In a launch of several rounds of waves
    // the oldest-first order lets the next round start sooner, so it is kept.)
    const bool prio = a.prio != 0;
    const int np = nfull >> 1;
    const int p1 = np >> 1, p2 = np - (np >> 2), p3 = np - (np >> 3);
    if (prio) __builtin_amdgcn_s_setprio(3);
    for (; g + 2 <= nfull; g += 2) {
      if (prio && (g >> 1) == p1) __builtin_amdgcn_s_setprio(2);
      if (prio && (g >> 1) == p2) __builtin_amdgcn_s_setprio(1);
      if (prio && (g >> 1) == p3) __builtin_amdgcn_s_setprio(0);
      code_group(g, NG, [&](int j) { return xa[j]; });
      load(xa, g + 2);
      code_group(g + 1, NG, [&](int j) { return xb[j]; });
      load(xb, g + 3);
    }
    if (g < nfull) code_group(g++, NG, [&](int j) { return xa[j]; });
  }
  for (; g < B.ng; g++) {
    const int ta = g * a.G;
    code_group(g, min(a.G, B.tc - ta),
               [&](int j) { return ld_half(xin, lane_off, (uint32_t)(ta + j) * row_bytes); });
  }
  if (B.tc > B.ng) {  // a stream without symbols stays empty
    rc_finish(e, o);
    flush_tail(o);
  }
  if (!(nfacc == 0.0f)) atomicOr(&B.status[2], 1u);
  const uint32_t nwords = sink_words(o);
  B.lens[(size_t)rrel * a.C + c] = nwords;
  reinterpret_cast<uint16_t*>(B.blob + B.lay.off_len)[pi] = (uint16_t)nwords;
}

// Anchor streams of coded-anchor blobs (payload rows 2L .. 4L-1): one lane
// per (kv, layer, channel), a workgroup per (group of up to 4 blobs, row,
// 64-channel block) with one wave per blob, as in k_encode.  The anchor of
// group g is chunk token g G, quantised as in the delta encoder's closed loop;
// its symbol a + 128 is range-coded with the (kv, layer) anchor table (CacheGen
// blog, section 2.1: the quantised anchor, then arithmetic coding), into the
// same per-block scratch layout as the delta streams, so the same kernels pack
// them.  Non-finite input is flagged by k_encode, which reads every token.
template <int RW>
__global__ __launch_bounds__(kLanes * kEncMaxWaves) void k_anchor_encode(EncodeArgs a) {
  uint32_t* cum = reinterpret_cast<uint32_t*>(enc_lds + (size_t)a.waves * RW * 256u);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int per_grp = a.nrows * a.nblk;
  const int grp = blockIdx.x / per_grp, unit = blockIdx.x % per_grp;
  const int rrel = unit / a.nblk;
  const int arow = a.row0 + rrel - 2 * a.L;  // kv * L + l
  const int cb = unit % a.nblk;
  if (wave == 0) {
    // cumulative table: lane k sums entries 4k .. 4k + 3, then a wave scan
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
  __syncthreads();
  const EncGroup& eg = a.groups[grp];
  const int bi = __builtin_amdgcn_readfirstlane(eg.blob[wave]);
  if (bi < 0) return;
  const EncBlob& B = a.b[bi];
  const int kv = arow / a.L, l = arow % a.L;
  const int c = cb * kLanes + lane;
  if (c >= a.C) return;
  const float inv_a = a.inv_a[(size_t)arow * a.C + c];
  // the chunk's rows of this (kv, layer), as in k_encode: no load may name a
  // row at or past tc (g G < tc for every group g)
  const uint32_t row_bytes = 2u * (uint32_t)a.C;
  const __amdgpu_buffer_rsrc_t xin = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((kv ? a.v : a.k) + ((size_t)l * a.T + B.t0) * a.C), 0,
      (int)((uint32_t)B.tc * row_bytes), kBufRsrcWord3);
  const uint32_t lane_off = 2u * (uint32_t)c;
  const size_t block = (size_t)rrel * a.nblk + cb;
  Sink<RW> o = make_sink<RW>(B.scratch + block * kLanes * a.swb, a.swb, (uint32_t)wave * RW * 256u, lane);
  RcEnc e = {0, 0u, 0xFFFFFFFFu, 0u, 0u, 0xFFFFFFFFu};
  const uint32_t gstep = (uint32_t)a.G * row_bytes;
  // anchor tokens in batches of kAB, loaded one batch ahead (a batch past the
  // last group re-reads the last group, inside the chunk)
  constexpr int kAB = 16;
  uint32_t xa[kAB], xb[kAB];
  auto load = [&](uint32_t (&x)[kAB], int g0) {
#pragma unroll
    for (int j = 0; j < kAB; j++) x[j] = ld_half(xin, lane_off, (uint32_t)min(g0 + j, B.ng - 1) * gstep);
  };
  auto code = [&](const uint32_t (&x)[kAB], int g0) {
#pragma unroll
    for (int j = 0; j < kAB; j++) {
      if (g0 + j >= B.ng) break;  // wave-uniform
      const uint32_t s = (uint32_t)(quant_anchor(half_bits_to_float(x[j]), inv_a) + 128);
      const uint32_t c0 = cum[s];
      rc_put(e, c0, cum[s + 1] - c0, o);
      flush_units(o);
    }
  };
  load(xa, 0);
  load(xb, kAB);
  for (int g0 = 0; g0 < B.ng; g0 += 2 * kAB) {
    code(xa, g0);
    load(xa, g0 + 2 * kAB);
    code(xb, g0 + kAB);
    load(xb, g0 + 3 * kAB);
  }
  rc_finish(e, o);  // every chunk has at least one group
  flush_tail(o);
  const uint32_t nwords = sink_words(o);
  B.lens[(size_t)rrel * a.C + c] = nwords;
  reinterpret_cast<uint16_t*>(B.blob + B.lay.off_len)[(size_t)(a.row0 + rrel) * a.C + c] =
      (uint16_t)nwords;
}

// words of every 64-stream block and of every payload row of the launch's
// range, for every blob
__global__ __launch_bounds__(256) void k_row_totals(EncodeArgs a) {
  __shared__ uint32_t part[4];
  const EncBlob& B = a.b[blockIdx.y];
  const int row = blockIdx.x, lane = threadIdx.x & 63;  // row within the range
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t* r = B.lens + (size_t)row * a.C;
  uint32_t total = 0;
  for (int cb = wave; cb < a.nblk; cb += 4) {
    const int c = cb * kLanes + lane;
    uint32_t s = c < a.C ? r[c] : 0u;
    for (int o = 32; o; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) B.block_words[(size_t)row * a.nblk + cb] = s;
    total += s;
  }
  if (lane == 0) part[wave] = total;
  __syncthreads();
  if (threadIdx.x == 0) B.row_words[row] = part[0] + part[1] + part[2] + part[3];
}

// per blob: offsets of the range's rows, continuing from the words of the rows
// coded before (a wavefront prefix sum, 64 rows at a time); flags a blob whose
// words so far do not fit cap (the range's packing is then skipped, and so is
// every later one); the launch that ends the rows writes the header and zeroes
// the padding (the gap before the payload and the tail after it)
__global__ __launch_bounds__(256) void k_row_scan(EncodeArgs a) {
  __shared__ uint32_t s_words, s_fits;
  const EncBlob& B = a.b[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63;
  const bool last = a.row0 + a.nrows == a.rows_total;
  if (tid < kLanes) {
    uint32_t* row_off = reinterpret_cast<uint32_t*>(B.blob + B.lay.off_rows);
    uint64_t w = B.status[0];
    for (int r0 = 0; r0 < a.nrows; r0 += kLanes) {
      const int r = r0 + lane;
      const uint32_t rw = r < a.nrows ? B.row_words[r] : 0u;
      uint64_t incl = rw;
      for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      if (r < a.nrows) row_off[a.row0 + r] = (uint32_t)(w + incl - rw);
      w += __shfl(incl, 63);
    }
    if (lane == 0) {
      const size_t total = blob_bytes(B.lay, w);
      const bool fits = total <= B.cap && w <= 0x3FFFFFFFull;
      B.status[0] = (uint32_t)w;
      if (!fits) B.status[1] = 1u;
      s_words = (uint32_t)w;
      s_fits = fits && B.status[1] == 0u ? 1u : 0u;
      if (last) {
        uint32_t* h = reinterpret_cast<uint32_t*>(B.blob);
        h[0] = kBlobMagic;
        h[1] = B.lay.off_anchor ? kBlobVersion : kBlobVersionCoded;
        h[2] = (uint32_t)a.L;
        h[3] = (uint32_t)a.C;
        h[4] = (uint32_t)a.T;
        h[5] = (uint32_t)B.t0;
        h[6] = (uint32_t)B.tc;
        h[7] = (uint32_t)a.G;
        h[8] = (uint32_t)B.ng;
        h[9] = (uint32_t)B.q;
        h[10] = (uint32_t)w;
        h[11] = kProbBits;
        h[12] = (uint32_t)a.tables_id;
        h[13] = (uint32_t)(a.tables_id >> 32);
        h[14] = 0;
        h[15] = 0;
      }
    }
  }
  __syncthreads();
  if (!last || !s_fits) return;
  const size_t W = s_words;
  const size_t gap0 = B.lay.off_len + 2 * (size_t)B.lay.rows * a.C, gap1 = B.lay.off_pay;
  const size_t tail0 = B.lay.off_pay + 4 * W, tail1 = blob_bytes(B.lay, W);
  for (size_t j = gap0 + tid; j < gap1; j += 256) B.blob[j] = 0;
  for (size_t j = tail0 + tid; j < tail1; j += 256) B.blob[j] = 0;
}

// Pack one 64-stream block into the payload layout: its payload offset is the
// row's offset plus the words of the row's earlier blocks; m = the fewest
// whole 16-byte units any of its streams has; units 0 .. m-1 of its ns streams
// first, unit by unit (unit u of stream j at word 4 (u ns + j)), then every
// stream's remaining words, stream after stream.  The block's words are in
// scratch as [unit][lane][4 words] already, so unit u of all its streams is one
// contiguous 16 ns-byte run there as in the payload; the tails are read a word
// at a time (the lanes are the streams).
__global__ __launch_bounds__(256) void k_pack(EncodeArgs a) {
  const EncBlob& B = a.b[blockIdx.y];
  if (B.status[1]) return;
  __shared__ uint32_t toff[kLanes], slen[kLanes];
  __shared__ uint32_t s_base, s_units, s_maxlen;
  const int rrel = blockIdx.x / a.nblk, cb = blockIdx.x % a.nblk;
  const int row = a.row0 + rrel;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ns = min(kLanes, a.C - cb * kLanes);
  if (wave == 0) {
    const uint32_t* bw = B.block_words + (size_t)rrel * a.nblk;
    uint32_t before = 0;
    for (int j = lane; j < cb; j += kLanes) before += bw[j];
    for (int o = 32; o; o >>= 1) before += __shfl_xor(before, o);
    const int c = cb * kLanes + lane;
    const uint32_t len = lane < ns ? B.lens[(size_t)rrel * a.C + c] : 0u;
    uint32_t mu = lane < ns ? len / 4u : 0xFFFFFFFFu, mx = len;
    for (int o = 32; o; o >>= 1) {
      mu = min(mu, __shfl_xor(mu, o));
      mx = max(mx, __shfl_xor(mx, o));
    }
    const uint32_t tl = lane < ns ? len - 4u * mu : 0u;  // this stream's tail words
    uint32_t incl = tl;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    toff[lane] = 4u * mu * (uint32_t)ns + incl - tl;
    slen[lane] = len;
    if (lane == 0) {
      s_base = reinterpret_cast<const uint32_t*>(B.blob + B.lay.off_rows)[row] + before;
      s_units = mu;
      s_maxlen = mx;
    }
  }
  __syncthreads();
  // the block's scratch: unit u of stream j (its words 4u .. 4u + 3) is the
  // 16 bytes at word 4 (64 u + j)
  const uint32_t* src = B.scratch + ((size_t)rrel * a.nblk + cb) * kLanes * a.swb;
  uint32_t* pay = reinterpret_cast<uint32_t*>(B.blob + B.lay.off_pay) + s_base;
  const uint32_t m = s_units, mx = s_maxlen;
  typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
  // interleaved units: wave w copies unit u = w, w + 4, ... of every stream
  if (lane < ns)
    for (uint32_t u = (uint32_t)wave; u < m; u += 4u)
      *reinterpret_cast<u32x4a*>(pay + 4u * (u * (uint32_t)ns + (uint32_t)lane)) =
          *reinterpret_cast<const u32x4a*>(src + 4u * (u * kLanes + (uint32_t)lane));
  // tails: stream j's words 4m .. len_j - 1
  for (uint32_t k = 4u * m + (uint32_t)wave; k < mx; k += 4u)
    if (lane < ns && k < slen[lane])
      pay[toff[lane] + (k - 4u * m)] = src[4u * ((k >> 2) * kLanes + (uint32_t)lane) + (k & 3u)];
}

}  // namespace

hipError_t launch_encode(const EncodeArgs& a, hipStream_t st) {
  const unsigned nb = (unsigned)a.nblobs;
  const unsigned blocks = (unsigned)(a.n_groups * a.nrows * a.nblk);
  // rings of 8 words where the launch's workgroups still fit their compute
  // units at once with them, else of 4
  const bool anc = a.row0 >= 2 * a.L;
  const size_t fixed = anc ? 4u * (kASym + 1) : 2u * kImgRows * kLanes;
  const size_t per_cu = (blocks + (unsigned)a.ncu - 1) / (unsigned)a.ncu;
  const bool r8 = per_cu * (fixed + (size_t)a.waves * 8u * 256u) <= (size_t)a.lds_cu;
  const size_t lds = fixed + (size_t)a.waves * (r8 ? 8u : 4u) * 256u;
  if (anc) {
    if (r8) k_anchor_encode<8><<<blocks, kLanes * a.waves, lds, st>>>(a);
    else k_anchor_encode<4><<<blocks, kLanes * a.waves, lds, st>>>(a);
  } else if (a.G == 10) {
    if (r8) k_encode<10, 8><<<blocks, kLanes * a.waves, lds, st>>>(a);
    else k_encode<10, 4><<<blocks, kLanes * a.waves, lds, st>>>(a);
  } else {
    if (r8) k_encode<0, 8><<<blocks, kLanes * a.waves, lds, st>>>(a);
    else k_encode<0, 4><<<blocks, kLanes * a.waves, lds, st>>>(a);
  }
  k_row_totals<<<dim3(a.nrows, nb), 256, 0, st>>>(a);
  k_row_scan<<<nb, 256, 0, st>>>(a);
  k_pack<<<dim3(a.nrows * a.nblk, nb), 256, 0, st>>>(a);
  return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(256) void k_zero_words(uint32_t* p, uint32_t n) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i < n) p[i] = 0u;
}
}  // namespace

hipError_t launch_zero_words(uint32_t* p, uint32_t n, hipStream_t st) {
  if (n) k_zero_words<<<(n + 255u) / 256u, 256, 0, st>>>(p, n);
  return hipGetLastError();
}

}  // namespace cg
