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
  const size_t pi = (size_t)row * a.C + (active ? c : 0);
  const float scale_a = a.scale_a[pi];
  const float step = a.step[q][pi];

  // start of this lane's stream: row offset + lengths of the streams before it
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
  const uint32_t start = ld32(rs, 64u + 4u * row) + before + incl - my_len;
  uint32_t bad = (active && (uint64_t)start + my_len > ch.W) ? 1u : 0u;

  // bit reader: `code` is the 32-bit window, `buf` the next 32..64 bits (most
  // significant first), `nxt` the word after them, already in flight
  uint32_t wof = ch.off_pay + 4u * start;
  uint32_t code = ld32(rs, wof);
  uint64_t buf = ((uint64_t)ld32(rs, wof + 4u) << 32) | ld32(rs, wof + 8u);
  uint32_t nxt = ld32(rs, wof + 12u);
  wof += 16u;
  int nb = 64;
  uint32_t range = 0xFFFFFFFFu;

  const uint8_t* tb = reinterpret_cast<const uint8_t*>(tab) + 2 * lane_slot(lane);
  uint16_t* out = (kv ? a.v_out : a.k_out) + ((size_t)l * a.T + ch.t0) * a.C + c;
  const uint32_t anc_base = ch.off_anchor + (uint32_t)row * (uint32_t)ch.ng * (uint32_t)a.C + c;

  for (int g = 0; g < ch.ng; g++) {
    const int ta = g * a.G, te = min(ta + a.G, ch.tc);
    const float ahat = anchor_value(ld8s(rs, anc_base + (uint32_t)g * a.C), scale_a);
    if (active) out[(size_t)ta * a.C] = float_to_half_bits(ahat);
    const float base = __builtin_fmaf(-32.0f, step, ahat);
    for (int t = ta + 1; t < te; t++) {
      const uint32_t r = range >> kProbBits;
      bad |= ((r << kProbBits) <= code) ? 1u : 0u;
      // largest s with r * cum[s] <= code, by bisection over the LDS column
      uint32_t s = 0;
#pragma unroll
      for (uint32_t stp = 32; stp; stp >>= 1) {
        const uint32_t key = *reinterpret_cast<const uint16_t*>(tb + (s + stp) * (2 * kLanes));
        if (mul24(r, key) <= code) s += stp;
      }
      const uint32_t c0 = *reinterpret_cast<const uint16_t*>(tb + s * (2 * kLanes));
      const uint32_t c1 = *reinterpret_cast<const uint16_t*>(tb + (s + 1) * (2 * kLanes));
      code -= mul24(r, c0);
      range = mul24(r, c1 - c0);
      // shift in whole bytes until range >= 2^24 (0, 1 or 2 bytes)
      const uint32_t sh = __clz(range) & 24u;
      const uint64_t win = ((uint64_t)code << 32) | (uint32_t)(buf >> 32);
      code = (uint32_t)((win << sh) >> 32);
      buf <<= sh;
      nb -= (int)sh;
      range <<= sh;
      if (nb <= 32) {
        buf |= (uint64_t)nxt << (32 - nb);
        nb += 32;
        nxt = ld32(rs, wof);
        wof += 4u;
      }
      if (active) out[(size_t)t * a.C] = float_to_half_bits(__builtin_fmaf((float)s, step, base));
    }
  }
  if (__any(bad & (active ? 1u : 0u))) {
    if (lane == 0) atomicOr(a.status, 1u);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)(a.n_groups * 2 * a.L * a.nblk);
  k_decode<<<blocks, kLanes * a.waves, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace cg
