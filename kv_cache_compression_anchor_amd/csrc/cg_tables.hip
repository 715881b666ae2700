// Table building on the GPU (CacheGen blog, section 1: symbol probabilities
// counted per layer-channel combination; section 2.1: step sizes 0.5/1.0/1.5 per
// layer group).  All reductions are exact integer sums, so the result does not
// depend on the order in which workgroups run.
#include <float.h>

#include "cg_build.h"

namespace cg {
namespace {

constexpr int kStatsRows = 1024;  // tokens per stats workgroup

// Exact moments of X = |x| * 2^24 for binary16 x.  A finite x is M * 2^(E-24)
// with M = m (+ 1024 when the exponent field e is not 0) and E = max(e - 1, 0),
// so X = M << E.  Each element adds only to its bucket, the binary16 bits
// 10..15 (sign and e): the packed word m + 2^20 (sum of m below bit 20, count
// above; a bucket sees at most 1024 elements) and m^2.  The buckets are folded
// into S1 = sum of signed X and S2 = sum of X^2 once per workgroup:
//   sum M = sum m + 1024 n,   sum M^2 = sum m^2 + 2048 sum m + 2^20 n   (e > 0).
// LDS: [64 buckets][packed | squares][64 lanes] u32.
constexpr int kStatsWords = 64 * 2 * kLanes;

__device__ __forceinline__ void stats_add(uint32_t* bk, uint32_t h, uint32_t lane4,
                                          uint32_t& amax) {
  const uint32_t ad = ((h >> 1) & 0x7E00u) | lane4;  // bucket * 512 + lane * 4
  uint32_t* p = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(bk) + ad);
  const uint32_t m = h & 0x3FFu;
  atomicAdd(p, m | 0x100000u);
  atomicAdd(p + kLanes, m * m);
  amax = max(amax, h & 0x7FFFu);
}

// One workgroup: 64 channels (a lane each) x kStatsRows tokens of one layer; the
// four waves take every fourth row, sixteen loads in flight per wave.
__global__ __launch_bounds__(256) void k_stats(const uint16_t* __restrict__ x, int kv, int L,
                                               int T, int C, StatsBuf sb) {
  __shared__ uint32_t bk[kStatsWords];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int j = tid; j < kStatsWords; j += 256) bk[j] = 0;
  __syncthreads();
  const int c = blockIdx.x * kLanes + lane;
  const int l = blockIdx.z;
  const int tbeg = blockIdx.y * kStatsRows;
  const int n = min(kStatsRows, T - tbeg);
  const uint32_t lane4 = 4u * (uint32_t)lane;
  uint32_t amax = 0;
  if (c < C) {
    const uint32_t row_bytes = 2u * (uint32_t)C;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + ((size_t)l * T + tbeg) * C + (size_t)blockIdx.x * kLanes), 0,
        (int)((uint32_t)n * row_bytes), kBufRsrcWord3);
    const uint32_t lane_off = 2u * (uint32_t)lane;
    int t = wave;
    constexpr int kU = 16;
    for (; t + 4 * (kU - 1) < n; t += 4 * kU) {
      uint32_t h[kU];
#pragma unroll
      for (int j = 0; j < kU; j++)
        h[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, lane_off, (uint32_t)(t + 4 * j) * row_bytes, 0);
#pragma unroll
      for (int j = 0; j < kU; j++) stats_add(bk, h[j], lane4, amax);
    }
    for (; t < n; t += 4)
      stats_add(bk, __builtin_amdgcn_raw_buffer_load_b16(rs, lane_off, (uint32_t)t * row_bytes, 0),
                lane4, amax);
  }
  __syncthreads();
  // fold: wave w takes buckets 16w .. 16w + 15 of its lane's channel
  int64_t s1 = 0;
  unsigned __int128 s2 = 0;
  for (int b = 16 * wave; b < 16 * wave + 16; b++) {
    const uint32_t e = (uint32_t)b & 31u;
    if (e == 31u) continue;  // infinities and NaNs: flagged through amax
    const uint32_t pk = bk[(b * 2) * kLanes + lane], sq = bk[(b * 2 + 1) * kLanes + lane];
    const uint64_t cnt = pk >> 20, sm = pk & 0xFFFFFu;
    const uint64_t SM = e ? sm + (cnt << 10) : sm;
    const uint64_t SQ = e ? (uint64_t)sq + (sm << 11) + (cnt << 20) : (uint64_t)sq;
    const uint32_t E = e ? e - 1u : 0u;
    const int64_t v = (int64_t)(SM << E);
    s1 += (b & 32) ? -v : v;
    s2 += (unsigned __int128)SQ << (2u * E);
  }
  __syncthreads();
  // the four waves' partials of each channel, summed by wave 0
  uint64_t* part = reinterpret_cast<uint64_t*>(bk);  // [wave][s1, sa, sc][lane]
  uint32_t* pmax = bk + 4 * 3 * kLanes * 2;          // [wave][lane]
  part[(wave * 3 + 0) * kLanes + lane] = (uint64_t)s1;
  part[(wave * 3 + 1) * kLanes + lane] = (uint64_t)(s2 >> 40);
  part[(wave * 3 + 2) * kLanes + lane] = (uint64_t)s2 & ((1ull << 40) - 1);
  pmax[wave * kLanes + lane] = amax;
  __syncthreads();
  if (wave != 0 || c >= C) return;
  uint64_t t1 = 0, ta = 0, tc = 0;
  uint32_t mx = 0;
  for (int w = 0; w < 4; w++) {
    t1 += part[(w * 3 + 0) * kLanes + lane];
    ta += part[(w * 3 + 1) * kLanes + lane];
    tc += part[(w * 3 + 2) * kLanes + lane];
    mx = max(mx, pmax[w * kLanes + lane]);
  }
  const size_t i0 = ((size_t)kv * L + l) * C + c;
  atomicAdd((unsigned long long*)&sb.s1[i0], (unsigned long long)t1);
  atomicAdd((unsigned long long*)&sb.sa[i0], (unsigned long long)ta);
  atomicAdd((unsigned long long*)&sb.sc[i0], (unsigned long long)tc);
  atomicMax(&sb.amax[i0], mx);
  if (mx >= 0x7C00u) atomicOr(&sb.flags[0], 1u);
}

// Correctly rounded (to nearest, ties to even) conversion of a 128-bit integer:
// keep the top 64 bits with the lost bits folded into a sticky bit, convert once.
__device__ double u128_to_f64(unsigned __int128 v) {
  const uint64_t hi = (uint64_t)(v >> 64);
  if (hi == 0) return (double)(uint64_t)v;
  const int shift = 64 - __clzll(hi);
  uint64_t top = (uint64_t)(v >> shift);
  const unsigned __int128 lost = v & (((unsigned __int128)1 << shift) - 1);
  top |= (lost != 0) ? 1ull : 0ull;
  return ldexp((double)top, shift);
}

struct FinArgs {
  StatsBuf sb;
  uint8_t* ser;
  int L, T, C;
  uint32_t mask;
  int lg_end[3];
  float layer_step[3];
  float mult[3];
  size_t off_scale_a, off_inv_a, off_step[3], off_inv_step[3];
};

// Population std over all tokens from the exact moments, anchor scale and the
// per-quality delta step of every (kv, layer, channel).
__global__ __launch_bounds__(256) void k_finalize(FinArgs a) {
  const size_t n = (size_t)2 * a.L * a.C;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int l = (int)((i / a.C) % a.L);
  const int64_t S1 = (int64_t)a.sb.s1[i];
  const unsigned __int128 S2 = ((unsigned __int128)a.sb.sa[i] << 40) + (unsigned __int128)a.sb.sc[i];
  const unsigned __int128 num =
      (unsigned __int128)a.T * S2 - (unsigned __int128)((__int128)S1 * S1);
  const double sigma = num ? sqrt(u128_to_f64(num)) / ((double)a.T * 16777216.0) : 1.0;
  const float amax = half_bits_to_float((uint16_t)a.sb.amax[i]);
  const float scale_a = amax > 0.0f ? (float)((double)amax / 127.0) : 1.0f;
  const float inv_a = (float)(1.0 / (double)scale_a);
  reinterpret_cast<float*>(a.ser + a.off_scale_a)[i] = scale_a;
  reinterpret_cast<float*>(a.ser + a.off_inv_a)[i] = inv_a;
  int g = 0;
  while (g < 2 && l >= a.lg_end[g]) g++;
  const double ls = (double)a.layer_step[g];
  for (int q = 0; q < 3; q++) {
    if (!((a.mask >> q) & 1u)) continue;
    const float step = (float)((double)a.mult[q] * ls * sigma);
    const float inv_step = (float)(1.0 / (double)step);
    if (!(step >= FLT_MIN) || !isfinite(inv_step)) atomicOr(&a.sb.flags[1], 1u);
    reinterpret_cast<float*>(a.ser + a.off_step[q])[i] = step;
    reinterpret_cast<float*>(a.ser + a.off_inv_step[q])[i] = inv_step;
  }
}

struct HistArgs {
  const uint16_t* x;
  int kv, L, T, C, CH, G, nq;
  const float* scale_a;
  const float* inv_a;
  const float* inv_step[3];  // by slot
  uint32_t* counts;          // [2][nq][L][C][64]
  uint32_t* acounts;         // [2][L][256] anchor-symbol counts, or null (raw anchors)
};

// Delta-symbol histogram of one (kv, layer, 64-channel block, chunk): each lane
// owns a channel, the four waves take interleaved groups; counts go to LDS with
// atomics, laid out [slot][symbol][lane] so that the 64 lanes hit distinct
// banks and a count's address is one shift-add of the delta level; then to
// global memory with one atomic per non-zero bin.  With coded anchors the
// anchors' symbols a + 128 are counted too, into 256 more LDS words.  LDS:
// nq * 16 KB (+ 1 KB), dynamic.
template <int GS, int NQ>
__global__ __launch_bounds__(256) void k_histogram(HistArgs a) {
  extern __shared__ uint32_t hist[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // token rows are scalar offsets
  const int words = NQ * kNSym * kLanes;
  const bool anchors = a.acounts != nullptr;
  uint32_t* ahist = hist + words;
  for (int j = tid; j < words + (anchors ? kASym : 0); j += 256) hist[j] = 0;
  __syncthreads();
  const int c = blockIdx.x * kLanes + lane;
  const int chunk = blockIdx.y, l = blockIdx.z;
  const int t0 = chunk * a.CH;
  const int tc = min(a.CH, a.T - t0);
  const int ng = (tc + a.G - 1) / a.G;
  if (c < a.C) {
    const size_t pi = ((size_t)a.kv * a.L + l) * a.C + c;
    const float scale_a = a.scale_a[pi], inv_a = a.inv_a[pi];
    const float is0 = a.inv_step[0][pi];
    const float is1 = NQ > 1 ? a.inv_step[1][pi] : 1.0f;
    const float is2 = NQ > 2 ? a.inv_step[2][pi] : 1.0f;
    // the chunk's rows of this layer: channel as the vector offset, token row as
    // a scalar offset.  The scalar offset is outside the buffer's range check,
    // so no load may name a row at or past tc.
    const uint32_t row_bytes = 2u * (uint32_t)a.C;
    const __amdgpu_buffer_rsrc_t xin = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.x + ((size_t)l * a.T + t0) * a.C), 0, (int)((uint32_t)tc * row_bytes),
        kBufRsrcWord3);
    const uint32_t lane_off = 2u * (uint32_t)c;
    auto ld = [&](int t) -> uint32_t {
      return __builtin_amdgcn_raw_buffer_load_b16(xin, lane_off, (uint32_t)t * row_bytes, 0);
    };
    // a count's byte address: level * 256 plus the slot column's address of
    // level 0, level = level_bits(u) - kLevelBias
    const uint32_t at0 = (uint32_t)(32 * kLanes + lane) * 4u - ((uint32_t)kLevelBias << 8);
    const uint32_t at1 = at0 + kNSym * kLanes * 4u, at2 = at1 + kNSym * kLanes * 4u;
    auto count = [&](uint32_t at, float u) {
      atomicAdd(reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(hist) +
                                            (((uint32_t)level_bits(u) << 8) + at)), 1u);
    };
    auto group = [&](int n, auto half_of) {
      const int av = quant_anchor(half_bits_to_float(half_of(0)), inv_a);
      if (anchors) atomicAdd(&ahist[av + 128], 1u);
      const float ahat = anchor_value(av, scale_a);
      for (int j = 1; j < n; j++) {
        const float d = half_bits_to_float(half_of(j)) - ahat;
        count(at0, d * is0);
        if constexpr (NQ > 1) count(at1, d * is1);
        if constexpr (NQ > 2) count(at2, d * is2);
      }
    };
    int g = wave;
    const int nfull = GS > 0 ? tc / GS : 0;
    if (GS > 0 && nfull > 0) {
      // full groups of the compile-time size, loaded one of this wave's groups
      // ahead (the loop issues only loads to memory, so the waits are exact).
      // A prefetch of a group past the last full one is never counted (the
      // loop ends first); it re-reads the last full group instead, so every
      // row read lies inside the chunk.
      constexpr int NG = GS > 0 ? GS : 1;
      uint32_t xa[NG], xb[NG];
      auto load = [&](uint32_t (&xv)[NG], int gg) {
        const int gl = min(gg, nfull - 1);
#pragma unroll
        for (int j = 0; j < NG; j++) xv[j] = ld(gl * NG + j);
      };
      load(xa, g);
      load(xb, g + 4);
      for (; g + 4 < nfull; g += 8) {
        group(NG, [&](int j) { return xa[j]; });
        load(xa, g + 8);
        group(NG, [&](int j) { return xb[j]; });
        load(xb, g + 12);
      }
      if (g < nfull) {
        group(NG, [&](int j) { return xa[j]; });
        g += 4;
      }
    }
    for (; g < ng; g += 4) {
      const int ta = g * a.G;
      group(min(a.G, tc - ta), [&](int j) { return ld(ta + j); });
    }
  }
  __syncthreads();
  for (int j = tid; j < words; j += 256) {
    const uint32_t v = hist[j];
    if (!v) continue;
    const int s = j / (kNSym * kLanes), sym = (j / kLanes) % kNSym, ln = j % kLanes;
    const int cc = blockIdx.x * kLanes + ln;
    const size_t ti = (((size_t)a.kv * NQ + s) * a.L + l) * a.C + cc;
    atomicAdd(&a.counts[ti * kNSym + sym], v);
  }
  if (anchors && tid < kASym && ahist[tid])
    atomicAdd(&a.acounts[((size_t)a.kv * a.L + l) * kASym + tid], ahist[tid]);
}

// Anchor tables: the counts of a (kv, layer) -> 256 frequencies summing to
// 2^15 by the same rule as the delta tables (one slot each, the rest in
// proportion rounded down, the remainder to the most counted symbol, lowest
// on ties).  One wave per table, lane k holds symbols k, k + 64, k + 128,
// k + 192.
__global__ __launch_bounds__(64) void k_normalize_anchors(const uint32_t* acounts, uint16_t* afreq) {
  const int k = threadIdx.x;
  const uint32_t* c = acounts + (size_t)blockIdx.x * kASym;
  uint32_t ck[4];
  uint64_t N = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    ck[j] = c[k + 64 * j];
    N += ck[j];
  }
  for (int o = 32; o; o >>= 1) N += __shfl_xor(N, o);
  const double spare = (double)(kProbTotal - kASym);
  const double den = N ? (double)N : (double)kASym;
  uint32_t f[4], total = 0, bc = 0, bk = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t cj = N ? ck[j] : 1u;
    // the floor of an exact quotient of integers below 2^47 and 2^32: the
    // correctly rounded binary64 quotient never crosses an integer
    f[j] = 1u + (uint32_t)floor((double)cj * spare / den);
    total += f[j];
    if (j == 0 || cj > bc) {  // this lane's most counted, lowest symbol on ties
      bc = cj;
      bk = (uint32_t)(k + 64 * j);
    }
  }
  for (int o = 32; o; o >>= 1) total += __shfl_xor(total, o);
  for (int o = 32; o; o >>= 1) {
    const uint32_t oc = __shfl_xor(bc, o), ok = __shfl_xor(bk, o);
    if (oc > bc || (oc == bc && ok < bk)) {
      bc = oc;
      bk = ok;
    }
  }
  uint16_t* out = afreq + (size_t)blockIdx.x * kASym;
#pragma unroll
  for (int j = 0; j < 4; j++)
    out[k + 64 * j] = (uint16_t)(f[j] + ((uint32_t)(k + 64 * j) == bk ? kProbTotal - total : 0u));
}

struct NormArgs {
  const uint32_t* counts;
  uint8_t* ser;
  int L, C, nq;
  int q_of_slot[3];
  size_t off_freq[3];
};

// counts -> frequencies summing to 2^15: one slot each, the rest in proportion
// (rounded down), the remainder to the most counted symbol (lowest on ties).
// One wave per table, one lane per symbol.
__global__ __launch_bounds__(256) void k_normalize(NormArgs a) {
  const size_t ntab = (size_t)2 * a.nq * a.L * a.C;
  const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int k = threadIdx.x & 63;
  if (i >= ntab) return;  // whole waves leave together
  const size_t lc = (size_t)a.L * a.C;
  const int kv = (int)(i / (a.nq * lc));
  const int s = (int)((i / lc) % a.nq);
  const size_t rest = i % lc;  // l * C + c
  const uint32_t c_k = a.counts[i * kNSym + k];
  uint64_t N = c_k;
  for (int o = 32; o; o >>= 1) N += __shfl_xor(N, o);
  const uint32_t ck = N ? c_k : 1u;
  const double spare = (double)(kProbTotal - kNSym);
  const double den = N ? (double)N : (double)kNSym;
  // floor of an exact quotient of integers below 2^36 and 2^22: the correctly
  // rounded binary64 quotient never crosses an integer
  uint32_t f = 1u + (uint32_t)floor((double)ck * spare / den);
  uint32_t total = f;
  for (int o = 32; o; o >>= 1) total += __shfl_xor(total, o);
  // the most counted symbol, lowest index on ties
  uint32_t bc = ck, bk = (uint32_t)k;
  for (int o = 32; o; o >>= 1) {
    const uint32_t oc = __shfl_xor(bc, o), ok = __shfl_xor(bk, o);
    if (oc > bc || (oc == bc && ok < bk)) {
      bc = oc;
      bk = ok;
    }
  }
  if ((uint32_t)k == bk) f += kProbTotal - total;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.ser + a.off_freq[a.q_of_slot[s]]) +
                  ((size_t)kv * lc + rest) * kNSym;
  out[k] = (uint16_t)f;
}

// Pooled symbol statistics (a coarser grouping than per layer and channel):
// grouping 1 sums the counts of a (kv, quality, layer) over its channels, 2 of
// a (kv, quality, channel) over its layers, 3 of a (kv, quality) over both;
// every member then takes the pooled counts, so its frequency table is the
// group's.  One thread per (kv, quality, group, symbol); a sum that does not
// fit 32 bits sets *overflow.
__global__ __launch_bounds__(256) void k_pool_sum(const uint32_t* counts, int L, int C, int nq,
                                                  int grouping, uint32_t* pooled,
                                                  uint32_t* overflow) {
  const int G = grouping == 1 ? L : grouping == 2 ? C : 1;
  const size_t n = (size_t)2 * nq * G * kNSym;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int sym = (int)(i % kNSym);
  const int g = (int)((i / kNSym) % G);
  const size_t ks = i / ((size_t)kNSym * G);  // kv * nq + slot
  const uint32_t* base = counts + ks * L * C * kNSym + sym;
  uint64_t sum = 0;
  if (grouping == 1) {
    for (int c = 0; c < C; c++) sum += base[((size_t)g * C + c) * kNSym];
  } else if (grouping == 2) {
    for (int l = 0; l < L; l++) sum += base[((size_t)l * C + g) * kNSym];
  } else {
    for (size_t j = 0; j < (size_t)L * C; j++) sum += base[j * kNSym];
  }
  if (sum > 0xFFFFFFFFull) atomicOr(overflow, 1u);
  pooled[i] = (uint32_t)sum;
}

__global__ __launch_bounds__(256) void k_pool_broadcast(uint32_t* counts, int L, int C, int nq,
                                                        int grouping, const uint32_t* pooled) {
  const int G = grouping == 1 ? L : grouping == 2 ? C : 1;
  const size_t n = (size_t)2 * nq * L * C * kNSym;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int sym = (int)(i % kNSym);
  const size_t tab = i / kNSym;  // ((kv * nq + slot) * L + l) * C + c
  const int c = (int)(tab % C);
  const int l = (int)((tab / C) % L);
  const size_t ks = tab / ((size_t)L * C);
  const int g = grouping == 1 ? l : grouping == 2 ? c : 0;
  counts[i] = pooled[(ks * G + g) * kNSym + sym];
}

struct ImgArgs {
  const uint8_t* ser;
  uint16_t* img[3];
  int L, C, nblk;
  size_t off_freq[3];
  uint32_t mask;
};

// Frequencies -> cumulative tables laid out as LDS images: per (kv, layer,
// 64-channel block) 65 rows of 64 16-bit entries, entry of lane j at
// lane_slot(j).  Channels past C get a uniform table.
__global__ __launch_bounds__(256) void k_images(ImgArgs a) {
  const size_t per_q = (size_t)2 * a.L * a.nblk * kLanes;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 3 * per_q) return;
  const int q = (int)(i / per_q);
  if (!((a.mask >> q) & 1u)) return;
  const size_t r = i % per_q;
  const int lane = (int)(r % kLanes);
  const size_t blk = r / kLanes;  // (kv * L + l) * nblk + cb
  const int cb = (int)(blk % a.nblk);
  const size_t row = blk / a.nblk;  // kv * L + l
  const int c = cb * kLanes + lane;
  uint16_t* out = a.img[q] + blk * (kImgRows * kLanes) + lane_slot(lane);
  uint32_t cum = 0;
  if (c < a.C) {
    const uint16_t* f =
        reinterpret_cast<const uint16_t*>(a.ser + a.off_freq[q]) + (row * a.C + c) * kNSym;
    for (int k = 0; k < kNSym; k++) {
      out[k * kLanes] = (uint16_t)cum;
      cum += f[k];
    }
  } else {
    for (int k = 0; k < kNSym; k++) {
      out[k * kLanes] = (uint16_t)cum;
      cum += kProbTotal / kNSym;
    }
  }
  out[kNSym * kLanes] = (uint16_t)cum;  // 2^15 does not fit 15 bits but fits 16
}

constexpr uint64_t kFnvBasis = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

__device__ __forceinline__ uint64_t fnv_byte(uint64_t h, uint32_t b) {
  return (h ^ b) * kFnvPrime;
}

// Tables id, a three-level FNV-1a-64 tree: digests of 1 KiB leaves (one thread
// each, 16-byte loads), digests of the little-endian bytes of 256 leaf digests,
// then the digest of the middle digests.
__global__ __launch_bounds__(256) void k_id_leaves(const uint8_t* ser, size_t n, uint64_t* d0) {
  const size_t n0 = (n + kIdLeaf - 1) / kIdLeaf;
  const size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n0) return;
  const size_t start = b * kIdLeaf;
  const size_t len = min((size_t)kIdLeaf, n - start);
  uint64_t h = kFnvBasis;
  size_t k = 0;
  if (len == (size_t)kIdLeaf) {  // full leaf: 16 bytes per load (ser is 256-byte aligned)
    const uint4* w = reinterpret_cast<const uint4*>(ser + start);
    for (; k < (size_t)kIdLeaf; k += 16) {
      const uint4 v = w[k / 16];
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        h = fnv_byte(h, q[j] & 0xFF);
        h = fnv_byte(h, (q[j] >> 8) & 0xFF);
        h = fnv_byte(h, (q[j] >> 16) & 0xFF);
        h = fnv_byte(h, q[j] >> 24);
      }
    }
  }
  for (; k < len; k++) h = fnv_byte(h, ser[start + k]);
  d0[b] = h;
}

__device__ __forceinline__ uint64_t fnv_digest(uint64_t h, uint64_t d) {
#pragma unroll
  for (int j = 0; j < 8; j++) h = fnv_byte(h, (uint32_t)(d >> (8 * j)) & 0xFF);
  return h;
}

__global__ __launch_bounds__(64) void k_id_mid(const uint64_t* d0, size_t n0, uint64_t* d1) {
  const size_t n1 = (n0 + kIdFan - 1) / kIdFan;
  const size_t j = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n1) return;
  const size_t end = min(n0, (j + 1) * (size_t)kIdFan);
  uint64_t h = kFnvBasis;
  for (size_t i = j * kIdFan; i < end; i++) h = fnv_digest(h, d0[i]);
  d1[j] = h;
}

__global__ void k_id_final(const uint64_t* d1, size_t n1, uint64_t* out) {
  uint64_t h = kFnvBasis;
  for (size_t j = 0; j < n1; j++) h = fnv_digest(h, d1[j]);
  *out = h;
}

inline unsigned blocks_for(size_t n, unsigned per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_stats(const uint16_t* x, int kv, int L, int T, int C, const StatsBuf& sb,
                        hipStream_t st) {
  dim3 grid((unsigned)((C + kLanes - 1) / kLanes), (unsigned)((T + kStatsRows - 1) / kStatsRows),
            (unsigned)L);
  k_stats<<<grid, 256, 0, st>>>(x, kv, L, T, C, sb);
  return hipGetLastError();
}

hipError_t launch_finalize(const cg_params& p, const StatsBuf& sb, DevTables& t, hipStream_t st) {
  FinArgs a;
  a.sb = sb;
  a.ser = t.ser;
  a.L = t.L;
  a.T = t.T;
  a.C = t.C;
  a.mask = t.mask;
  for (int g = 0; g < 3; g++) {
    a.lg_end[g] = g < p.n_layer_groups ? p.layer_group_end[g] : t.L;
    a.layer_step[g] = g < p.n_layer_groups ? p.layer_step[g] : p.layer_step[p.n_layer_groups - 1];
    a.mult[g] = p.quality_mult[g];
    a.off_step[g] = t.lay.off_step[g];
    a.off_inv_step[g] = t.lay.off_inv_step[g];
  }
  a.off_scale_a = t.lay.off_scale_a;
  a.off_inv_a = t.lay.off_inv_a;
  k_finalize<<<blocks_for(t.lay.n, 256), 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_histogram(const uint16_t* x, int kv, const DevTables& t, uint32_t* counts,
                            uint32_t* acounts, hipStream_t st) {
  HistArgs a;
  a.x = x;
  a.kv = kv;
  a.L = t.L;
  a.T = t.T;
  a.C = t.C;
  a.CH = t.CH;
  a.G = t.G;
  a.nq = t.lay.nq;
  a.scale_a = reinterpret_cast<const float*>(t.ser + t.lay.off_scale_a);
  a.inv_a = reinterpret_cast<const float*>(t.ser + t.lay.off_inv_a);
  for (int q = 0, s = 0; q < 3; q++)
    if ((t.mask >> q) & 1u) a.inv_step[s++] = reinterpret_cast<const float*>(t.ser + t.lay.off_inv_step[q]);
  a.counts = counts;
  a.acounts = t.lay.off_afreq ? acounts : nullptr;
  const int nchunks = (t.T + t.CH - 1) / t.CH;
  dim3 grid((unsigned)t.nblk, (unsigned)nchunks, (unsigned)t.L);
  const size_t lds = (size_t)a.nq * kNSym * kLanes * 4 + (a.acounts ? 4 * kASym : 0);
  const bool g10 = t.G == 10;
  if (a.nq == 1) {
    if (g10) k_histogram<10, 1><<<grid, 256, lds, st>>>(a);
    else k_histogram<0, 1><<<grid, 256, lds, st>>>(a);
  } else if (a.nq == 2) {
    if (g10) k_histogram<10, 2><<<grid, 256, lds, st>>>(a);
    else k_histogram<0, 2><<<grid, 256, lds, st>>>(a);
  } else {
    if (g10) k_histogram<10, 3><<<grid, 256, lds, st>>>(a);
    else k_histogram<0, 3><<<grid, 256, lds, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_normalize_anchors(const DevTables& t, const uint32_t* acounts, hipStream_t st) {
  if (!t.lay.off_afreq) return hipSuccess;
  k_normalize_anchors<<<2 * t.L, 64, 0, st>>>(acounts,
                                             reinterpret_cast<uint16_t*>(t.ser + t.lay.off_afreq));
  return hipGetLastError();
}

hipError_t launch_normalize(const DevTables& t, const uint32_t* counts, hipStream_t st) {
  NormArgs a;
  a.counts = counts;
  a.ser = t.ser;
  a.L = t.L;
  a.C = t.C;
  a.nq = t.lay.nq;
  for (int q = 0, s = 0; q < 3; q++) {
    a.off_freq[q] = t.lay.off_freq[q];
    if ((t.mask >> q) & 1u) a.q_of_slot[s++] = q;
  }
  const size_t ntab = (size_t)2 * a.nq * t.L * t.C;
  k_normalize<<<blocks_for(ntab * kLanes, 256), 256, 0, st>>>(a);
  return hipGetLastError();
}

size_t pooled_words(const DevTables& t, int grouping) {
  const int G = grouping == 1 ? t.L : grouping == 2 ? t.C : 1;
  return (size_t)2 * t.lay.nq * G * kNSym;
}

hipError_t launch_pool(const DevTables& t, uint32_t* counts, int grouping, uint32_t* pooled,
                       uint32_t* overflow, hipStream_t st) {
  const size_t np = pooled_words(t, grouping);
  k_pool_sum<<<blocks_for(np, 256), 256, 0, st>>>(counts, t.L, t.C, t.lay.nq, grouping, pooled,
                                                  overflow);
  const size_t n = (size_t)2 * t.lay.nq * t.L * t.C * kNSym;
  k_pool_broadcast<<<blocks_for(n, 256), 256, 0, st>>>(counts, t.L, t.C, t.lay.nq, grouping,
                                                       pooled);
  return hipGetLastError();
}

hipError_t launch_images(DevTables& t, hipStream_t st) {
  ImgArgs a;
  a.ser = t.ser;
  for (int q = 0; q < 3; q++) {
    a.img[q] = t.img[q];
    a.off_freq[q] = t.lay.off_freq[q];
  }
  a.L = t.L;
  a.C = t.C;
  a.nblk = t.nblk;
  a.mask = t.mask;
  const size_t n = (size_t)3 * 2 * t.L * t.nblk * kLanes;
  k_images<<<blocks_for(n, 256), 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_tables_id(const DevTables& t, uint64_t* digests, uint64_t* id_out,
                            hipStream_t st) {
  const size_t n0 = id_leaves(t.lay.total), n1 = id_mids(t.lay.total);
  k_id_leaves<<<blocks_for(n0, 256), 256, 0, st>>>(t.ser, t.lay.total, digests);
  k_id_mid<<<blocks_for(n1, 64), 64, 0, st>>>(digests, n0, digests + n0);
  k_id_final<<<1, 1, 0, st>>>(digests + n0, n1, id_out);
  return hipGetLastError();
}

}  // namespace cg
