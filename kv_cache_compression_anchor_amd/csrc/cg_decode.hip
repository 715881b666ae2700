// Chunk decoder (gptget 方法详解: the receiver decodes the bitstream on the GPU;
// CacheGen blog, section 2.1: anchor plus delta reconstruction).
//
// One lane per stream (kv, layer, channel), one wave per chunk, one workgroup
// per (group of chunks with the same quality, kv, layer, 64-channel block): the
// workgroup stages the block's 64 cumulative tables in LDS once and every wave
// decodes its chunk against them.  All lanes of a wave sit on the same token,
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

__device__ __forceinline__ uint32_t lds16(const uint8_t* base, uint32_t byte_off) {
  return *reinterpret_cast<const uint16_t*>(base + byte_off);
}

// Row stride of an LDS table image: entry k of every lane lives in row k.
constexpr uint32_t kRow = 2 * kLanes;

__global__ __launch_bounds__(256) void k_decode(DecodeArgs a) {
  __shared__ uint16_t tab[kImgRows * kLanes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per_grp = 2 * a.L * a.nblk;
  const int grp = blockIdx.x / per_grp, rem = blockIdx.x % per_grp;
  const int kv = rem / (a.L * a.nblk), l = (rem / a.nblk) % a.L, cb = rem % a.nblk;
  const int row = kv * a.L + l;
  const int q = a.chunks[a.groups[grp].chunk[0]].q;
  {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(
        a.img[q] + ((size_t)row * a.nblk + cb) * (kImgRows * kLanes));
    uint32_t* dst = reinterpret_cast<uint32_t*>(tab);
    for (int j = tid; j < kImgRows * kLanes / 2; j += blockDim.x) dst[j] = src[j];
  }
  __syncthreads();
  const int ci = a.groups[grp].chunk[wave];
  if (ci < 0) return;
  const DecChunk ch = a.chunks[ci];
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)ch.blob, 0, (int)ch.blob_bytes, kBufRsrcWord3);

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
  const float step_row = step * (1.0f / kRow);  // exact: a power-of-two scaling

  const uint8_t* tb = reinterpret_cast<const uint8_t*>(tab);
  const uint32_t lane_addr = 2u * lane_slot(lane);      // LDS byte address of cum[0]
  const uint32_t key32 = lds16(tb, lane_addr + 32u * kRow);  // root of the search, kept in a register

  // bit reader: `code` is the 32-bit window, b1:b0 the next nb bits (most
  // significant first; 32..64 before every pair of symbols), `nxt` the word
  // after them, already in flight
  uint32_t wof = ch.off_pay + 4u * start;
  uint32_t code = ld32(rs, wof);
  uint32_t b1 = ld32(rs, wof + 4u), b0 = ld32(rs, wof + 8u);
  uint32_t nxt = ld32(rs, wof + 12u);
  wof += 16u;
  int nb = 64;
  uint32_t range = 0xFFFFFFFFu;

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
    // largest s with r * cum[s] <= code; `ad` is the LDS address of cum[s]
    uint32_t ad = (mul24(r, key32) <= code) ? lane_addr + 32u * kRow : lane_addr;
#pragma unroll
    for (uint32_t stp = 16; stp; stp >>= 1) {
      if (mul24(r, lds16(tb, ad + stp * kRow)) <= code) ad += stp * kRow;
    }
    const uint32_t lo = mul24(r, lds16(tb, ad));
    const uint32_t hi = mul24(r, lds16(tb, ad + kRow));
    code -= lo;
    range = hi - lo;
    // shift in whole bytes until range >= 2^24 (0, 1 or 2 bytes; range > 0)
    const uint32_t sh = (uint32_t)__builtin_clz(range) & 24u;
    const uint64_t w_hi = ((uint64_t)code << 32) | b1;
    const uint64_t w_lo = (((uint64_t)b1 << 32) | b0) << sh;
    code = (uint32_t)((w_hi << sh) >> 32);
    b1 = (uint32_t)(w_lo >> 32);
    b0 = (uint32_t)w_lo;
    nb -= (int)sh;
    range <<= sh;
    // (ad - lane_addr) = s * kRow, so this is fma(s, step, base) exactly
    const float y = __builtin_fmaf((float)(ad - lane_addr), step_row, base);
    __builtin_amdgcn_raw_buffer_store_b16(float_to_half_bits(y), ro, lane_off, soff, 0);
  };

  for (int g = 0; g < ch.ng; g++) {
    const int ta = g * a.G, te = min(ta + a.G, ch.tc);
    const int anc = anc_next;
    if (g + 1 < ch.ng) anc_next = ld8s(rs, anc_base + (uint32_t)(g + 1) * a.C);
    const float ahat = anchor_value(anc, scale_a);
    __builtin_amdgcn_raw_buffer_store_b16(float_to_half_bits(ahat), ro, lane_off,
                                          (uint32_t)ta * row_bytes, 0);
    const float base = __builtin_fmaf(-32.0f, step, ahat);
    for (int t = ta + 1; t < te; t += 2) {
      // at least 32 buffered bits cover the next two symbols (16 bits each at most)
      if (nb < 32) {
        const uint64_t add = (uint64_t)nxt << (32 - nb);
        b1 |= (uint32_t)(add >> 32);
        b0 |= (uint32_t)add;
        nb += 32;
        nxt = ld32(rs, wof);
        wof += 4u;
      }
      symbol((uint32_t)t * row_bytes, base);
      if (t + 1 < te) symbol((uint32_t)(t + 1) * row_bytes, base);
    }
  }
  // a valid stream keeps code < range throughout; a corrupt one breaks it for good
  bad |= (code >= range) ? 1u : 0u;
  if (bad) atomicOr(a.status, 1u);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)(a.n_groups * 2 * a.L * a.nblk);
  k_decode<<<blocks, kLanes * a.waves, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace cg
