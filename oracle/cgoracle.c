/*
 * CPU oracle of the CacheGen KV-cache tensor codec — TEST INFRASTRUCTURE ONLY.
 * Plain scalar C: no blocking, fusion or reordering beyond what each step states.
 * Floating point is IEEE binary32 (SSE, no FMA contraction: build with
 * -ffp-contract=off) except where a step says binary64 or fmaf.
 * Parallelism (OpenMP) is only across independent (kv, layer) rows.
 *
 * Sources: CacheGen (arXiv 2310.07240) as summarised on the gptget page
 * (方法详解), the sciencestack page (TL;DR, Figures 3-5) and the CacheGen blog
 * (section 1, the section 2.1 pseudocode, section 2.2).  The pages fix: groups
 * of ten tokens with the first as an 8-bit anchor and deltas against it; delta
 * steps 0.5 / 1.0 / 1.5 for shallow / medium / deep layers; arithmetic coding
 * with probability tables per (layer, channel); 1.5K-token chunks; H/M/L
 * quality versions.  Everything else below is a reading of those passages.
 */
#include "cgoracle.h"

#include <fenv.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define NSYM 64                 /* delta symbols -32..31, offset by 32 */
#define PBITS 15                /* probability precision: freqs sum to 2^15 */
#define PTOT 32768u
#define RC_TOP (1u << 24)       /* renormalise while range < 2^24 */
#define TAB_HDR 80
#define BLOB_HDR 64
#define TAB_MAGIC 0x31544743u   /* "CGT1" */
#define BLOB_MAGIC 0x314B4743u  /* "CGK1" */
#define BLOB_VERSION 2          /* payload blocks laid out as below (stream_layout) */
#define BLOB_VERSION_CODED 3    /* the same with range-coded anchors (reading R14) */
#define TAB_VERSION 1           /* tables without anchor tables */
#define TAB_VERSION_CODED 2     /* tables with one anchor table per (kv, layer) */
#define ASYM 256                /* anchor symbols: value a in -127..127 is a + 128 */
#define BLOCK_STREAMS 64        /* streams per payload block */
#define UNIT_WORDS 4            /* a 16-byte unit of a stream */
#define MAX_TOKENS (1 << 21)
#define MAX_CHUNK 65536

enum { OK = 0, E_INVAL = -1, E_NOMEM = -2, E_CORRUPT = -4, E_CAPACITY = -5, E_MISMATCH = -6 };

/* ------------------------------------------------------------------------- */
/* IEEE 754 binary16                                                          */
/* ------------------------------------------------------------------------- */

/* binary16 -> binary32 from the format definition: sign, 5-bit biased
 * exponent (bias 15), 10-bit fraction; exponent 0 is subnormal, 31 is Inf/NaN. */
float cgo_f16_to_f32(uint16_t h) {
  int e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0)
    v = ldexpf((float)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexpf((float)(m + 1024), e - 25);
  return (h & 0x8000) ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even, from the definition:
 * the result is the binary16 value nearest |f|; magnitudes from 65520 up (the
 * midpoint between 65504 and 2^16) overflow to infinity. */
uint16_t cgo_f32_to_f16(float f) {
  uint16_t sign = (signbit(f) ? 0x8000 : 0);
  if (isnan(f)) return sign | 0x7E00;
  double a = fabs((double)f);
  if (a >= 65520.0) return sign | 0x7C00;
  if (a < ldexp(1.0, -14)) {               /* subnormal range, quantum 2^-24 */
    double n = nearbyint(a * 16777216.0);  /* exact scaling; ties to even */
    return sign | (uint16_t)n;             /* n == 1024 is the least normal */
  }
  int e2;
  frexp(a, &e2);
  int E = e2 - 1;                          /* a in [2^E, 2^(E+1)) */
  double n = nearbyint(ldexp(a, 10 - E));  /* 11-bit significand, [1024, 2048] */
  if (n == 2048.0) { n = 1024.0; E += 1; }
  if (E > 15) return sign | 0x7C00;
  return sign | (uint16_t)(((E + 15) << 10) | ((int)n - 1024));
}

void cgo_f16_to_f32_array(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = cgo_f16_to_f32(in[i]);
}
void cgo_f32_to_f16_array(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = cgo_f32_to_f16(in[i]);
}

/* ------------------------------------------------------------------------- */
/* Range coder (arithmetic coding with integer ranges).                       */
/* The pages name arithmetic coding (gptget 方法详解; sciencestack TL;DR;     */
/* CacheGen blog 2.1 "arithmetic_encode").  Reading: a 32-bit range coder     */
/* with carry propagation, byte renormalisation below 2^24, frequencies of    */
/* 15 bits; the flush leaves a codeword that decodes correctly whatever bytes */
/* follow it.                                                                 */
/* ------------------------------------------------------------------------- */

size_t cgo_rc_bound(int64_t n) {
  if (n <= 0) return 0;
  /* each symbol costs < 15.003 bits; the flush adds at most two bytes */
  return (size_t)((n * 15 + n / 256 + 7) / 8) + 4;
}

static int make_cum(const uint16_t* freq, int nsym, uint32_t* cum) {
  if (nsym < 1 || nsym > 256) return E_INVAL;
  cum[0] = 0;
  for (int s = 0; s < nsym; s++) cum[s + 1] = cum[s] + freq[s];
  return cum[nsym] == PTOT ? OK : E_INVAL;
}

/* add one to the byte string out[0..m), as a big-endian number */
static int propagate_carry(uint8_t* out, size_t m) {
  size_t i = m;
  while (i > 0) {
    i--;
    if (out[i] == 0xFF) {
      out[i] = 0;
    } else {
      out[i]++;
      return OK;
    }
  }
  return E_CORRUPT; /* impossible: the coded value stays below 1 */
}

int cgo_rc_encode(const uint8_t* sym, int64_t n, const uint16_t* freq, int nsym,
                  uint8_t* out, size_t cap, size_t* out_len) {
  uint32_t cum[257];
  if (make_cum(freq, nsym, cum) != OK) return E_INVAL;
  *out_len = 0;
  if (n <= 0) return OK; /* a stream without symbols is empty */
  if (cap < cgo_rc_bound(n)) return E_CAPACITY;
  uint64_t low = 0;              /* bottom of the interval, current 32-bit window */
  uint32_t range = 0xFFFFFFFFu;  /* width of the interval */
  size_t m = 0;
  for (int64_t i = 0; i < n; i++) {
    int s = sym[i];
    if (s >= nsym || freq[s] == 0) return E_INVAL;
    uint32_t r = range >> PBITS;
    low += (uint64_t)r * cum[s];
    range = r * freq[s];
    if (low >> 32) { /* the interval moved past the window: carry into the output */
      low &= 0xFFFFFFFFu;
      if (propagate_carry(out, m) != OK) return E_CORRUPT;
    }
    while (range < RC_TOP) {
      out[m++] = (uint8_t)(low >> 24);
      low = (low << 8) & 0xFFFFFFFFu;
      range <<= 8;
    }
  }
  /* flush: the fewest bytes (1 or 2) naming an aligned block inside [low, low+range) */
  int k;
  uint64_t V = 0;
  for (k = 1; k <= 2; k++) {
    uint64_t q = 1ull << (32 - 8 * k);
    V = (low + q - 1) / q * q;
    if (V + q <= low + range) break;
  }
  if (k > 2) return E_CORRUPT; /* impossible with range >= 2^24 */
  if (V >> 32) {
    V &= 0xFFFFFFFFu;
    if (propagate_carry(out, m) != OK) return E_CORRUPT;
  }
  out[m++] = (uint8_t)(V >> 24);
  if (k == 2) out[m++] = (uint8_t)(V >> 16);
  *out_len = m;
  return OK;
}

/* Decoder: bytes at buf[i] for i >= buflen read as zero (the caller appends the
 * real continuation when it matters).  The symbol is the largest s with
 * r*cum[s] <= code, found by a linear scan from the top. */
int cgo_rc_decode(const uint8_t* buf, size_t buflen, int64_t n, const uint16_t* freq,
                  int nsym, uint8_t* sym, size_t* consumed, int* corrupt) {
  uint32_t cum[257];
  if (make_cum(freq, nsym, cum) != OK) return E_INVAL;
  size_t pos = 0;
  if (n <= 0) {
    if (consumed) *consumed = 0;
    return OK;
  }
#define NEXT_BYTE() ((uint32_t)(pos < buflen ? buf[pos] : 0))
  uint32_t code = 0;
  for (int i = 0; i < 4; i++) { code = (code << 8) | NEXT_BYTE(); pos++; }
  uint32_t range = 0xFFFFFFFFu;
  for (int64_t i = 0; i < n; i++) {
    uint32_t r = range >> PBITS;
    if ((uint64_t)r * PTOT <= code) *corrupt = 1; /* code outside every symbol */
    int s = nsym - 1;
    while (s > 0 && (freq[s] == 0 || (uint64_t)r * cum[s] > code)) s--;
    sym[i] = (uint8_t)s;
    code -= r * cum[s];
    range = r * freq[s];
    if (range == 0) { *corrupt = 1; range = 1u << 31; }
    while (range < RC_TOP) {
      code = (code << 8) | NEXT_BYTE();
      pos++;
      range <<= 8;
    }
  }
#undef NEXT_BYTE
  if (consumed) *consumed = pos;
  return OK;
}

/* Frequency table from symbol counts (reading of "symbol probabilities counted
 * per layer-channel combination", CacheGen blog section 1): every symbol gets
 * at least 1/2^15 so any symbol stays codable; the rest is shared in
 * proportion to the counts, rounded down; the remainder goes to the most
 * frequent symbol (lowest index on ties).  No counts at all counts as one of each. */
void cgo_normalize(const uint32_t* counts, int nsym, uint16_t* freq) {
  uint64_t N = 0;
  for (int s = 0; s < nsym; s++) N += counts[s];
  uint64_t spare = PTOT - (uint64_t)nsym;
  uint32_t total = 0;
  int best = 0;
  for (int s = 0; s < nsym; s++) {
    uint64_t c = N ? counts[s] : 1;
    uint64_t den = N ? N : (uint64_t)nsym;
    freq[s] = (uint16_t)(1 + c * spare / den);
    total += freq[s];
    uint64_t cb = N ? counts[best] : 1;
    if (c > cb) best = s;
  }
  freq[best] = (uint16_t)(freq[best] + (PTOT - total));
}

/* ntab consecutive tables of NSYM counts each */
void cgo_normalize_tables(const uint32_t* counts, int64_t ntab, uint16_t* freq) {
  for (int64_t i = 0; i < ntab; i++) cgo_normalize(counts + i * NSYM, NSYM, freq + i * NSYM);
}

/* ------------------------------------------------------------------------- */
/* Channel statistics                                                         */
/* ------------------------------------------------------------------------- */

/* x * 2^24 as an exact integer, for a finite binary16 x */
static int64_t f16_scaled_int(uint16_t h) {
  int e = (h >> 10) & 31, m = h & 1023;
  int64_t X = e ? ((int64_t)(m + 1024) << (e - 1)) : (int64_t)m;
  return (h & 0x8000) ? -X : X;
}

/* Population standard deviation over all tokens of every (l, c), exactly:
 * with X = x*2^24, num = N*sum(X^2) - (sum X)^2 in 128-bit integers, then
 * sigma = sqrt(num) / (N * 2^24) in binary64; a zero deviation reads as 1.
 * This is the "channel std" unit of the delta step. */
void cgo_channel_stats(const uint16_t* x, int L, int T, int C, double* sigma,
                       float* absmax, int* nonfinite) {
  int nf = 0;
  /* integer sums do not depend on the order of the terms: layers run in
   * parallel, tokens in order with one accumulator per channel */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : nf)
  for (int l = 0; l < L; l++) {
    int64_t* S1 = (int64_t*)calloc(C, sizeof(int64_t));
    unsigned __int128* S2 = (unsigned __int128*)calloc(C, sizeof(unsigned __int128));
    uint16_t* amax = (uint16_t*)calloc(C, sizeof(uint16_t));
    for (int t = 0; t < T; t++) {
      const uint16_t* row = x + ((size_t)l * T + t) * C;
      for (int c = 0; c < C; c++) {
        uint16_t h = row[c];
        if (((h >> 10) & 31) == 31) { nf = 1; continue; }
        int64_t X = f16_scaled_int(h);
        S1[c] += X;
        S2[c] += (unsigned __int128)((__int128)X * X);
        if ((h & 0x7FFF) > amax[c]) amax[c] = h & 0x7FFF;
      }
    }
    for (int c = 0; c < C; c++) {
      unsigned __int128 num = (unsigned __int128)T * S2[c] -
                              (unsigned __int128)((__int128)S1[c] * S1[c]);
      sigma[(size_t)l * C + c] = num ? sqrt((double)num) / ((double)T * 16777216.0) : 1.0;
      absmax[(size_t)l * C + c] = cgo_f16_to_f32(amax[c]);
    }
    free(S1);
    free(S2);
    free(amax);
  }
  *nonfinite = nf;
}

/* ------------------------------------------------------------------------- */
/* Quantisation (CacheGen blog, section 2.1 pseudocode: the group's first     */
/* token is quantised to 8 bits, the other nine are deltas against it).       */
/* ------------------------------------------------------------------------- */

/* anchor: symmetric 8-bit code against the channel's absolute maximum */
static int8_t quant_anchor(float x, float inv_a) {
  float p = x * inv_a;
  float r = rintf(p);
  if (r < -127.0f) r = -127.0f;
  if (r > 127.0f) r = 127.0f;
  return (int8_t)r;
}

static float anchor_value(int8_t a, float scale_a) { return (float)a * scale_a; }

/* delta against the reconstructed anchor, in steps, clipped to [-32, 31] */
static uint8_t quant_delta(float x, float ahat, float inv_step) {
  float d = x - ahat;
  float u = d * inv_step;
  float r = rintf(u);
  if (r < -32.0f) r = -32.0f;
  if (r > 31.0f) r = 31.0f;
  return (uint8_t)((int)r + 32);
}

/* The error-free sum of two binary64 values (Knuth's TwoSum): s + *err equals
 * a + b exactly, s being the binary64 sum rounded to nearest. */
static double two_sum(double a, double b, double* err) {
  double s = a + b;
  double bp = s - a;
  double ap = s - bp;
  *err = (a - ap) + (b - bp);
  return s;
}

/* Bits of a non-negative value that binary16 represents exactly (65536, one
 * past the largest finite value, is infinity). */
static uint16_t f16_bits_exact(double v) {
  if (v >= 65536.0) return 0x7C00;
  if (v < ldexp(1.0, -14)) return (uint16_t)(v * 16777216.0); /* subnormal: v / 2^-24 */
  int e2;
  double m = frexp(v, &e2);                                      /* v = m 2^e2, m in [0.5, 1) */
  return (uint16_t)(((e2 - 1 + 15) << 10) | ((int)ldexp(m, 11) - 1024));
}

/* The binary16 value nearest to the real number S + e, ties to even, where S
 * is binary64 and e the exact error of the binary64 sum that gave S (so e is
 * at most half a binary64 ulp of S and S + e is the exact value).  Written
 * from the format's definition: the magnitude |S + e| lies between two
 * consecutive multiples n q and (n + 1) q of the binary16 quantum q of its
 * binade (2^-24 below 2^-14); the nearer one is taken, and at the midpoint the
 * sign of e decides, or, when e is zero, the even n. */
static uint16_t f16_nearest(double S, double e) {
  uint16_t sign = 0;
  if (S < 0.0 || (S == 0.0 && e < 0.0)) {
    sign = 0x8000;
    S = -S;
    e = -e;
  }
  if (S > 65520.0 || (S == 65520.0 && e >= 0.0)) return sign | 0x7C00; /* past 65504's half-way */
  double q;
  if (S < ldexp(1.0, -14)) {
    q = ldexp(1.0, -24);
  } else {
    int e2;
    frexp(S, &e2);                 /* S in [2^(e2-1), 2^e2) */
    q = ldexp(1.0, e2 - 1 - 10);
  }
  double n = floor(S / q);         /* S / q is an exact scaling */
  double rem = S - n * q;          /* exact: both are multiples of S's binary64 ulp */
  double half = q / 2.0;
  int up = rem > half || (rem == half && (e > 0.0 || (e == 0.0 && fmod(n, 2.0) == 1.0)));
  return sign | f16_bits_exact((n + (up ? 1.0 : 0.0)) * q);
}

/* Reconstruction of a delta token (CacheGen blog, section 2.1: deltas are taken
 * against the quantised anchor): the binary16 value nearest to the exact real
 * number ahat + (s - 32) * step, ties to even.  (s - 32) * step is exact in
 * binary64 (6 by 24 significant bits); the sum's rounding error is carried
 * along exactly. */
static uint16_t dequant_delta(uint8_t s, float step, float ahat) {
  double p = (double)((int)s - 32) * (double)step;
  double err;
  double S = two_sum((double)ahat, p, &err);
  return f16_nearest(S, err);
}

void cgo_dequant_delta_array(const uint8_t* s, const float* step, const float* ahat,
                             uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = dequant_delta(s[i], step[i], ahat[i]);
}

/* ------------------------------------------------------------------------- */
/* Tables                                                                     */
/* ------------------------------------------------------------------------- */

static uint32_t rd32(const uint8_t* p) { uint32_t v; memcpy(&v, p, 4); return v; }
static int32_t rdi32(const uint8_t* p) { int32_t v; memcpy(&v, p, 4); return v; }
static uint64_t rd64(const uint8_t* p) { uint64_t v; memcpy(&v, p, 8); return v; }
static float rdf(const uint8_t* p) { float v; memcpy(&v, p, 4); return v; }
static void wr32(uint8_t* p, uint32_t v) { memcpy(p, &v, 4); }
static void wri32(uint8_t* p, int32_t v) { memcpy(p, &v, 4); }
static void wr64(uint8_t* p, uint64_t v) { memcpy(p, &v, 8); }
static void wrf(uint8_t* p, float v) { memcpy(p, &v, 4); }

uint64_t cgo_fnv1a64(const uint8_t* data, size_t n) {
  uint64_t h = 0xcbf29ce484222325ull;
  for (size_t i = 0; i < n; i++) {
    h ^= data[i];
    h *= 0x100000001b3ull;
  }
  return h;
}

/* Identity of a serialized table set, stamped into every blob (a digest of
 * the codebook, which the pages leave to the implementation): a three-level
 * FNV-1a-64 tree.  Leaves are the digests of consecutive 1 KiB blocks (the last
 * may be shorter); each middle digest covers the little-endian bytes of up to
 * 256 consecutive leaf digests; the id is the digest of the little-endian
 * middle digests. */
#define ID_LEAF 1024
#define ID_FAN 256
static uint64_t fnv1a64_of_digests(const uint64_t* d, size_t n) {
  uint8_t* b = (uint8_t*)malloc(8 * (n ? n : 1));
  for (size_t i = 0; i < n; i++)
    for (int j = 0; j < 8; j++) b[8 * i + j] = (uint8_t)(d[i] >> (8 * j));
  uint64_t h = cgo_fnv1a64(b, 8 * n);
  free(b);
  return h;
}
uint64_t cgo_tables_id(const uint8_t* data, size_t n) {
  size_t n0 = (n + ID_LEAF - 1) / ID_LEAF;
  size_t n1 = (n0 + ID_FAN - 1) / ID_FAN;
  uint64_t* d0 = (uint64_t*)malloc(8 * (n0 ? n0 : 1));
  uint64_t* d1 = (uint64_t*)malloc(8 * (n1 ? n1 : 1));
  for (size_t i = 0; i < n0; i++) {
    size_t len = (n - ID_LEAF * i < ID_LEAF) ? n - ID_LEAF * i : ID_LEAF;
    d0[i] = cgo_fnv1a64(data + ID_LEAF * i, len);
  }
  for (size_t j = 0; j < n1; j++) {
    size_t cnt = (n0 - ID_FAN * j < ID_FAN) ? n0 - ID_FAN * j : ID_FAN;
    d1[j] = fnv1a64_of_digests(d0 + ID_FAN * j, cnt);
  }
  uint64_t id = fnv1a64_of_digests(d1, n1);
  free(d0);
  free(d1);
  return id;
}

static int nq_of(uint32_t mask) { return (mask & 1) + ((mask >> 1) & 1) + ((mask >> 2) & 1); }

static int check_params(const cgo_params* p) {
  if (p->layers < 1 || p->tokens < 1 || p->channels < 1) return E_INVAL;
  if (p->tokens > MAX_TOKENS || p->channels > 65536 || p->layers > 4096) return E_INVAL;
  if (p->chunk_tokens < 1 || p->chunk_tokens > MAX_CHUNK) return E_INVAL;
  if (p->group_tokens < 1 || p->group_tokens > p->chunk_tokens) return E_INVAL;
  if (p->n_layer_groups < 1 || p->n_layer_groups > 3) return E_INVAL;
  int prev = 0;
  for (int i = 0; i < p->n_layer_groups; i++) {
    if (p->layer_group_end[i] <= prev) return E_INVAL;
    prev = p->layer_group_end[i];
    if (!(p->layer_step[i] > 0.0f) || !isfinite(p->layer_step[i])) return E_INVAL;
  }
  if (prev != p->layers) return E_INVAL;
  if ((p->quality_mask & ~7u) || !p->quality_mask) return E_INVAL;
  if (p->anchor_coding != 0 && p->anchor_coding != 1) return E_INVAL;
  /* an anchor table counts channels x groups per layer: at most C x T < 2^32 */
  if (p->anchor_coding && (uint64_t)p->channels * (uint64_t)p->tokens >= (1ull << 32))
    return E_INVAL;
  for (int q = 0; q < 3; q++)
    if ((p->quality_mask >> q) & 1)
      if (!(p->quality_mult[q] > 0.0f) || !isfinite(p->quality_mult[q])) return E_INVAL;
  return OK;
}

size_t cgo_tables_size(const cgo_params* p) {
  size_t n = (size_t)2 * p->layers * p->channels;
  return TAB_HDR + 8 * n + (size_t)nq_of(p->quality_mask) * (8 * n + 2 * NSYM * n) +
         (p->anchor_coding ? (size_t)2 * p->layers * ASYM * 2 : 0);
}

static int layer_group(const cgo_params* p, int l) {
  for (int i = 0; i < p->n_layer_groups; i++)
    if (l < p->layer_group_end[i]) return i;
  return p->n_layer_groups - 1;
}

/* parsed view of a serialized table set */
typedef struct {
  cgo_params p;
  size_t n;                  /* 2*L*C */
  const uint8_t* scale_a;    /* f32 [2][L][C] */
  const uint8_t* inv_a;
  const uint8_t* step[3];    /* f32 [2][L][C] per quality (NULL if absent) */
  const uint8_t* inv_step[3];
  const uint8_t* freq[3];    /* u16 [2][L][C][64] */
  const uint8_t* afreq;      /* u16 [2][L][256] anchor tables (NULL: raw anchors) */
  uint64_t id;
} tabview;

static int parse_tables(const uint8_t* t, size_t len, tabview* tv) {
  if (len < TAB_HDR || rd32(t) != TAB_MAGIC) return E_INVAL;
  uint32_t version = rd32(t + 4);
  if (version != TAB_VERSION && version != TAB_VERSION_CODED) return E_INVAL;
  cgo_params* p = &tv->p;
  p->anchor_coding = version == TAB_VERSION_CODED;
  p->layers = rdi32(t + 8);
  p->channels = rdi32(t + 12);
  p->tokens = rdi32(t + 16);
  p->chunk_tokens = rdi32(t + 20);
  p->group_tokens = rdi32(t + 24);
  p->n_layer_groups = rdi32(t + 28);
  for (int i = 0; i < 3; i++) {
    p->layer_group_end[i] = rdi32(t + 32 + 4 * i);
    p->layer_step[i] = rdf(t + 44 + 4 * i);
    p->quality_mult[i] = rdf(t + 56 + 4 * i);
  }
  p->quality_mask = rd32(t + 68);
  if (rd32(t + 72) != PBITS || rd32(t + 76) != NSYM) return E_INVAL;
  if (check_params(p) != OK) return E_INVAL;
  if (cgo_tables_size(p) != len) return E_INVAL;
  tv->n = (size_t)2 * p->layers * p->channels;
  const uint8_t* q = t + TAB_HDR;
  tv->scale_a = q; q += 4 * tv->n;
  tv->inv_a = q; q += 4 * tv->n;
  for (int k = 0; k < 3; k++) {
    tv->step[k] = tv->inv_step[k] = tv->freq[k] = NULL;
    if (!((p->quality_mask >> k) & 1)) continue;
    tv->step[k] = q; q += 4 * tv->n;
    tv->inv_step[k] = q; q += 4 * tv->n;
    tv->freq[k] = q; q += 2 * NSYM * tv->n;
  }
  tv->afreq = p->anchor_coding ? q : NULL;
  tv->id = cgo_tables_id(t, len);
  return OK;
}

static float tv_f(const uint8_t* base, size_t i) { return rdf(base + 4 * i); }
static void tv_freq(const uint8_t* base, size_t i, uint16_t* f) {
  memcpy(f, base + 2 * NSYM * i, 2 * NSYM);
}

/* delta-symbol counts of one [L][T][C] tensor at one quality, per (l, c), over
 * every chunk and group, anchors excluded */
static void count_symbols(const cgo_params* p, const uint16_t* x, const float* scale_a,
                          const float* inv_a, const float* inv_step, int nthreads,
                          uint32_t* counts) {
  const int L = p->layers, T = p->tokens, C = p->channels;
  const int CH = p->chunk_tokens, G = p->group_tokens;
  memset(counts, 0, sizeof(uint32_t) * NSYM * (size_t)L * C);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int l = 0; l < L; l++) {
    float* ahat = (float*)malloc(sizeof(float) * C);
    for (int t0 = 0; t0 < T; t0 += CH) {
      int tc = (T - t0 < CH) ? T - t0 : CH;
      for (int g0 = 0; g0 < tc; g0 += G) {
        int ge = (g0 + G < tc) ? g0 + G : tc;
        const uint16_t* row = x + ((size_t)l * T + t0 + g0) * C;
        for (int c = 0; c < C; c++) {
          size_t i = (size_t)l * C + c;
          ahat[c] = anchor_value(quant_anchor(cgo_f16_to_f32(row[c]), inv_a[i]), scale_a[i]);
        }
        for (int t = g0 + 1; t < ge; t++) {
          const uint16_t* r = x + ((size_t)l * T + t0 + t) * C;
          for (int c = 0; c < C; c++) {
            size_t i = (size_t)l * C + c;
            uint8_t s = quant_delta(cgo_f16_to_f32(r[c]), ahat[c], inv_step[i]);
            counts[i * NSYM + s]++;
          }
        }
      }
    }
    free(ahat);
  }
}

/* anchor-symbol counts of one [L][T][C] tensor, per layer over every chunk,
 * group and channel (reading R14: one anchor table per (kv, layer), counted
 * over the tensor the tables are built from; anchors do not depend on the
 * quality) */
static void count_anchors(const cgo_params* p, const uint16_t* x, const float* inv_a,
                          uint32_t* counts) {
  const int L = p->layers, T = p->tokens, C = p->channels;
  const int CH = p->chunk_tokens, G = p->group_tokens;
  memset(counts, 0, sizeof(uint32_t) * ASYM * (size_t)L);
  for (int l = 0; l < L; l++)
    for (int t0 = 0; t0 < T; t0 += CH) {
      int tc = (T - t0 < CH) ? T - t0 : CH;
      for (int g0 = 0; g0 < tc; g0 += G) {
        const uint16_t* row = x + ((size_t)l * T + t0 + g0) * C;
        for (int c = 0; c < C; c++) {
          int a = quant_anchor(cgo_f16_to_f32(row[c]), inv_a[(size_t)l * C + c]);
          counts[(size_t)l * ASYM + a + 128]++;
        }
      }
    }
}

int cgo_build_tables(const cgo_params* p, const uint16_t* k, const uint16_t* v,
                     int nthreads, uint8_t* out, size_t cap, size_t* len,
                     uint32_t* counts_out) {
  if (check_params(p) != OK) return E_INVAL;
  size_t size = cgo_tables_size(p);
  if (cap < size) return E_CAPACITY;
  if (nthreads <= 0) nthreads = 1;
  const int L = p->layers, C = p->channels;
  const size_t lc = (size_t)L * C, n = 2 * lc;
  double* sigma = (double*)malloc(sizeof(double) * n);
  float* amax = (float*)malloc(sizeof(float) * n);
  float* scale_a = (float*)malloc(sizeof(float) * n);
  float* inv_a = (float*)malloc(sizeof(float) * n);
  float* step = (float*)malloc(sizeof(float) * n);
  float* inv_step = (float*)malloc(sizeof(float) * n);
  uint32_t* counts = (uint32_t*)malloc(sizeof(uint32_t) * NSYM * n);
  if (!sigma || !amax || !scale_a || !inv_a || !step || !inv_step || !counts) {
    free(sigma); free(amax); free(scale_a); free(inv_a); free(step); free(inv_step);
    free(counts);
    return E_NOMEM;
  }
  int rc = OK;
  for (int kv = 0; kv < 2 && rc == OK; kv++) {
    int nf = 0;
    cgo_channel_stats(kv ? v : k, L, p->tokens, C, sigma + kv * lc, amax + kv * lc, &nf);
    if (nf) rc = E_INVAL; /* non-finite input cannot be profiled */
  }
  if (rc != OK) goto done;
  for (size_t i = 0; i < n; i++) {
    /* 8-bit anchor scale: absmax / 127 in binary64, rounded to binary32 */
    scale_a[i] = amax[i] > 0.0f ? (float)((double)amax[i] / 127.0) : 1.0f;
    inv_a[i] = (float)(1.0 / (double)scale_a[i]);
  }
  memset(out, 0, size);
  wr32(out, TAB_MAGIC);
  wr32(out + 4, p->anchor_coding ? TAB_VERSION_CODED : TAB_VERSION);
  wri32(out + 8, p->layers);
  wri32(out + 12, p->channels);
  wri32(out + 16, p->tokens);
  wri32(out + 20, p->chunk_tokens);
  wri32(out + 24, p->group_tokens);
  wri32(out + 28, p->n_layer_groups);
  for (int i = 0; i < 3; i++) {
    wri32(out + 32 + 4 * i, i < p->n_layer_groups ? p->layer_group_end[i] : 0);
    wrf(out + 44 + 4 * i, i < p->n_layer_groups ? p->layer_step[i] : 0.0f);
    wrf(out + 56 + 4 * i, ((p->quality_mask >> i) & 1) ? p->quality_mult[i] : 0.0f);
  }
  wr32(out + 68, p->quality_mask);
  wr32(out + 72, PBITS);
  wr32(out + 76, NSYM);
  uint8_t* w = out + TAB_HDR;
  for (size_t i = 0; i < n; i++) wrf(w + 4 * i, scale_a[i]);
  w += 4 * n;
  for (size_t i = 0; i < n; i++) wrf(w + 4 * i, inv_a[i]);
  w += 4 * n;
  for (int q = 0; q < 3; q++) {
    if (!((p->quality_mask >> q) & 1)) continue;
    for (int kv = 0; kv < 2; kv++)
      for (int l = 0; l < L; l++) {
        /* step = quality multiplier x layer-group step x channel std (blog 2.1) */
        double ls = (double)p->layer_step[layer_group(p, l)];
        for (int c = 0; c < C; c++) {
          size_t i = kv * lc + (size_t)l * C + c;
          step[i] = (float)((double)p->quality_mult[q] * ls * sigma[i]);
          inv_step[i] = (float)(1.0 / (double)step[i]);
        }
      }
    for (size_t i = 0; i < n; i++) {
      if (!(step[i] >= 1.1754943508222875e-38f) || !isfinite(inv_step[i])) {
        rc = E_INVAL; /* step not a normal binary32 */
        goto done;
      }
    }
    for (int kv = 0; kv < 2; kv++)
      count_symbols(p, kv ? v : k, scale_a + kv * lc, inv_a + kv * lc, inv_step + kv * lc,
                    nthreads, counts + kv * lc * NSYM);
    if (counts_out) {
      int qi = 0;
      for (int j = 0; j < q; j++) qi += (p->quality_mask >> j) & 1;
      memcpy(counts_out + (size_t)qi * n * NSYM, counts, sizeof(uint32_t) * NSYM * n);
    }
    for (size_t i = 0; i < n; i++) wrf(w + 4 * i, step[i]);
    w += 4 * n;
    for (size_t i = 0; i < n; i++) wrf(w + 4 * i, inv_step[i]);
    w += 4 * n;
    for (size_t i = 0; i < n; i++) {
      uint16_t f[NSYM];
      cgo_normalize(counts + i * NSYM, NSYM, f);
      memcpy(w + 2 * NSYM * i, f, 2 * NSYM);
    }
    w += 2 * NSYM * n;
  }
  if (p->anchor_coding) {
    uint32_t* ac = (uint32_t*)malloc(sizeof(uint32_t) * ASYM * L);
    if (!ac) {
      rc = E_NOMEM;
      goto done;
    }
    for (int kv = 0; kv < 2; kv++) {
      count_anchors(p, kv ? v : k, inv_a + kv * lc, ac);
      for (int l = 0; l < L; l++) {
        uint16_t f[ASYM];
        cgo_normalize(ac + (size_t)l * ASYM, ASYM, f);
        memcpy(w, f, 2 * ASYM);
        w += 2 * ASYM;
      }
    }
    free(ac);
  }
  *len = size;
done:
  free(sigma); free(amax); free(scale_a); free(inv_a); free(step); free(inv_step);
  free(counts);
  return rc;
}

/* ------------------------------------------------------------------------- */
/* Chunk blobs                                                                */
/* ------------------------------------------------------------------------- */

static size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

/* Blob container offsets (readings R13, R14).  Raw anchors (version 2):
 * header, u32 row_offset[2L], i8 anchors[2][L][ng][C], u16 lengths[2L][C],
 * pad to 16, payload.  Coded anchors (version 3): header, u32 row_offset[4L],
 * u16 lengths[4L][C], pad to 16, payload; rows 0 .. 2L-1 hold the delta
 * streams of (kv, layer) = (r / L, r % L), rows 2L .. 4L-1 the anchor streams
 * of (kv, layer) = ((r - 2L) / L, (r - 2L) % L). */
typedef struct {
  int rows;  /* payload rows */
  size_t off_anchor, off_len, off_pay;
} blobgeo;

static blobgeo blob_geometry(int L, int C, int ng, int coded) {
  blobgeo g;
  g.rows = coded ? 4 * L : 2 * L;
  size_t after_rows = BLOB_HDR + 4 * (size_t)g.rows;
  g.off_anchor = coded ? 0 : after_rows;
  g.off_len = coded ? after_rows : after_rows + 2 * (size_t)L * ng * C;
  g.off_pay = align16(g.off_len + 2 * (size_t)g.rows * C);
  return g;
}

int cgo_chunk_geometry(const uint8_t* tables, size_t tlen, int chunk, int32_t* t0,
                       int32_t* tc, int32_t* n_groups) {
  tabview tv;
  if (parse_tables(tables, tlen, &tv) != OK) return E_INVAL;
  int CH = tv.p.chunk_tokens, T = tv.p.tokens, G = tv.p.group_tokens;
  int nchunks = (T + CH - 1) / CH;
  if (chunk < 0 || chunk >= nchunks) return E_INVAL;
  *t0 = chunk * CH;
  *tc = (T - *t0 < CH) ? T - *t0 : CH;
  *n_groups = (*tc + G - 1) / G;
  return OK;
}

/* stream capacity for one (kv, l, c) of a chunk with tc tokens, in 32-bit words */
static size_t stream_words_bound(int tc, int ng) {
  return (cgo_rc_bound(tc - ng) + 3) / 4;
}

size_t cgo_encode_bound(const uint8_t* tables, size_t tlen, int chunk) {
  tabview tv;
  int32_t t0, tc, ng;
  if (parse_tables(tables, tlen, &tv) != OK) return 0;
  if (cgo_chunk_geometry(tables, tlen, chunk, &t0, &tc, &ng) != OK) return 0;
  size_t L = tv.p.layers, C = tv.p.channels;
  const blobgeo geo = blob_geometry((int)L, (int)C, ng, tv.afreq != NULL);
  size_t words = 2 * L * C * stream_words_bound(tc, ng);
  if (tv.afreq) words += 2 * L * C * ((cgo_rc_bound(ng) + 3) / 4);
  return align16(geo.off_pay + 4 * words + 16);
}

/* a binary16 value whose exponent field is all ones is infinite or NaN */
static int any_nonfinite(const uint16_t* x, size_t stride, int n) {
  for (int t = 0; t < n; t++)
    if ((x[(size_t)t * stride] & 0x7C00) == 0x7C00) return 1;
  return 0;
}

/* symbols of one channel of one chunk: anchors[g] and delta symbols in token
 * order (the group's first token is the anchor, the others are deltas) */
static void channel_symbols(const uint16_t* x, size_t stride, int tc, int G, float scale_a,
                            float inv_a, float inv_step, int8_t* anchors, uint8_t* sym,
                            uint8_t* per_token) {
  int ns = 0, g = 0;
  for (int g0 = 0; g0 < tc; g0 += G, g++) {
    int ge = (g0 + G < tc) ? g0 + G : tc;
    int8_t a = quant_anchor(cgo_f16_to_f32(x[(size_t)g0 * stride]), inv_a);
    float ahat = anchor_value(a, scale_a);
    anchors[g] = a;
    if (per_token) per_token[g0] = 255;
    for (int t = g0 + 1; t < ge; t++) {
      uint8_t s = quant_delta(cgo_f16_to_f32(x[(size_t)t * stride]), ahat, inv_step);
      if (sym) sym[ns++] = s;
      if (per_token) per_token[t] = s;
    }
  }
}

/* bytes -> big-endian 32-bit words, zero padded */
static size_t bytes_to_words(const uint8_t* b, size_t nb, uint32_t* w) {
  size_t nw = (nb + 3) / 4;
  for (size_t i = 0; i < nw; i++) {
    uint32_t v = 0;
    for (int j = 0; j < 4; j++) v = (v << 8) | (4 * i + j < nb ? b[4 * i + j] : 0);
    w[i] = v;
  }
  return nw;
}

/* Payload layout (reading R13).  The streams of a (kv, layer) row lie in
 * blocks of BLOCK_STREAMS consecutive channels (the last block may hold fewer),
 * blocks one after another.  Inside a block of ns streams of len[0..ns) words,
 * m = the fewest whole 16-byte units (UNIT_WORDS words) any of its streams has;
 * units 0 .. m-1 of the ns streams come first, unit by unit (unit u of stream
 * j is the four words at 4 (u ns + j)), then every stream's remaining words,
 * 4m .. len[j]-1, stream after stream.  Nothing is padded: the block holds
 * exactly the sum of its streams' words. */
static int block_units(const uint16_t* len, int ns) {
  int m = 0;
  for (int j = 0; j < ns; j++) {
    int u = len[j] / UNIT_WORDS;
    if (j == 0 || u < m) m = u;
  }
  return m;
}

/* tail[j] = offset in the block of stream j's first word past its first m units */
static void block_tails(const uint16_t* len, int ns, int m, size_t* tail) {
  size_t off = (size_t)UNIT_WORDS * m * ns;
  for (int j = 0; j < ns; j++) {
    tail[j] = off;
    off += len[j] - (size_t)UNIT_WORDS * m;
  }
}

/* offset in the block of word w of stream j */
static size_t block_word(int ns, int m, const size_t* tail, int j, size_t w) {
  if (w < (size_t)UNIT_WORDS * m)
    return UNIT_WORDS * ((w / UNIT_WORDS) * ns + j) + w % UNIT_WORDS;
  return tail[j] + (w - (size_t)UNIT_WORDS * m);
}

/* the row's streams (each one's words consecutive in `src`, lengths `len`,
 * C channels) into the payload layout at `dst` */
static void lay_out_row(const uint32_t* src, const uint16_t* len, int C, uint32_t* dst) {
  size_t base = 0, s = 0;
  size_t tail[BLOCK_STREAMS];
  for (int c0 = 0; c0 < C; c0 += BLOCK_STREAMS) {
    int ns = C - c0 < BLOCK_STREAMS ? C - c0 : BLOCK_STREAMS;
    int m = block_units(len + c0, ns);
    block_tails(len + c0, ns, m, tail);
    size_t words = 0;
    for (int j = 0; j < ns; j++) {
      for (size_t w = 0; w < len[c0 + j]; w++) dst[base + block_word(ns, m, tail, j, w)] = src[s + w];
      s += len[c0 + j];
      words += len[c0 + j];
    }
    base += words;
  }
}

int cgo_encode_chunk(const uint8_t* tables, size_t tlen, const uint16_t* k,
                     const uint16_t* v, int chunk, int q, int nthreads, uint8_t* out,
                     size_t cap, size_t* len) {
  tabview tv;
  int32_t t0, tc, ng;
  if (parse_tables(tables, tlen, &tv) != OK) return E_INVAL;
  if (q < 0 || q > 2 || !tv.freq[q]) return E_MISMATCH;
  if (cgo_chunk_geometry(tables, tlen, chunk, &t0, &tc, &ng) != OK) return E_INVAL;
  if (nthreads <= 0) nthreads = 1;
  const int L = tv.p.layers, C = tv.p.channels, T = tv.p.tokens, G = tv.p.group_tokens;
  const int coded = tv.afreq != NULL;
  const size_t lc = (size_t)L * C;
  const int nsyms = tc - ng;
  const size_t swb = stream_words_bound(tc, ng);
  const size_t aswb = (cgo_rc_bound(ng) + 3) / 4;
  const blobgeo geo = blob_geometry(L, C, ng, coded);
  const int R = geo.rows;
  /* per row: words of every stream, then concatenated in row order */
  uint32_t** rows = (uint32_t**)calloc(R, sizeof(uint32_t*));
  uint32_t* rowlen = (uint32_t*)calloc(R, sizeof(uint32_t));
  uint16_t* slen = (uint16_t*)calloc((size_t)R * C, sizeof(uint16_t));
  int8_t* anchors = (int8_t*)calloc(2 * (size_t)L * ng * C, 1);
  if (!rows || !rowlen || !slen || !anchors) {
    free(rows); free(rowlen); free(slen); free(anchors);
    return E_NOMEM;
  }
  int rc = OK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int row = 0; row < 2 * L; row++) {
    int kv = row / L, l = row % L;
    const uint16_t* x = (kv ? v : k) + ((size_t)l * T + t0) * C;
    uint32_t* buf = (uint32_t*)malloc(sizeof(uint32_t) * (swb * C + 1));
    uint32_t* abuf = coded ? (uint32_t*)malloc(sizeof(uint32_t) * (aswb * C + 1)) : NULL;
    uint8_t* sym = (uint8_t*)malloc(nsyms + 1);
    uint8_t* bytes = (uint8_t*)malloc(cgo_rc_bound(nsyms > ng ? nsyms : ng) + 1);
    int8_t* anc = (int8_t*)malloc(ng);
    uint8_t* asym = (uint8_t*)malloc(ng);
    if (!buf || (coded && !abuf) || !sym || !bytes || !anc || !asym) {
#pragma omp critical
      rc = E_NOMEM;
      free(buf); free(abuf); free(sym); free(bytes); free(anc); free(asym);
      continue;
    }
    size_t used = 0, aused = 0;
    for (int c = 0; c < C; c++) {
      size_t i = kv * lc + (size_t)l * C + c;
      if (any_nonfinite(x + c, C, tc)) {
#pragma omp critical
        rc = E_INVAL; /* non-finite input cannot be coded */
      }
      uint16_t f[NSYM];
      tv_freq(tv.freq[q], i, f);
      channel_symbols(x + c, C, tc, G, tv_f(tv.scale_a, i), tv_f(tv.inv_a, i),
                      tv_f(tv.inv_step[q], i), anc, sym, NULL);
      for (int g = 0; g < ng; g++) anchors[(((size_t)kv * L + l) * ng + g) * C + c] = anc[g];
      size_t nb = 0;
      int e = cgo_rc_encode(sym, nsyms, f, NSYM, bytes, cgo_rc_bound(nsyms) + 1, &nb);
      if (e != OK) {
#pragma omp critical
        rc = e;
      }
      size_t nw = bytes_to_words(bytes, nb, buf + used);
      slen[(size_t)row * C + c] = (uint16_t)nw;
      used += nw;
      if (coded) {
        /* the anchor stream: symbol a + 128 of every group, with the (kv, layer)
         * anchor table (reading R14) */
        uint16_t af[ASYM];
        memcpy(af, tv.afreq + 2 * ASYM * ((size_t)kv * L + l), sizeof(af));
        for (int g = 0; g < ng; g++) asym[g] = (uint8_t)(anc[g] + 128);
        e = cgo_rc_encode(asym, ng, af, ASYM, bytes, cgo_rc_bound(ng) + 1, &nb);
        if (e != OK) {
#pragma omp critical
          rc = e;
        }
        nw = bytes_to_words(bytes, nb, abuf + aused);
        slen[(size_t)(2 * L + row) * C + c] = (uint16_t)nw;
        aused += nw;
      }
    }
    rows[row] = buf;
    rowlen[row] = (uint32_t)used;
    if (coded) {
      rows[2 * L + row] = abuf;
      rowlen[2 * L + row] = (uint32_t)aused;
    }
    free(sym); free(bytes); free(anc); free(asym);
  }
  size_t W = 0;
  for (int r = 0; r < R; r++) W += rowlen[r];
  size_t total = align16(geo.off_pay + 4 * W + 16);
  if (rc == OK && total > cap) rc = E_CAPACITY;
  if (rc == OK) {
    memset(out, 0, total);
    wr32(out, BLOB_MAGIC);
    wr32(out + 4, coded ? BLOB_VERSION_CODED : BLOB_VERSION);
    wri32(out + 8, L);
    wri32(out + 12, C);
    wri32(out + 16, T);
    wri32(out + 20, t0);
    wri32(out + 24, tc);
    wri32(out + 28, G);
    wri32(out + 32, ng);
    wri32(out + 36, q);
    wr32(out + 40, (uint32_t)W);
    wr32(out + 44, PBITS);
    wr64(out + 48, tv.id);
    size_t woff = 0, most = 0;
    for (int r = 0; r < R; r++)
      if (rowlen[r] > most) most = rowlen[r];
    uint32_t* laid = (uint32_t*)malloc(sizeof(uint32_t) * (most + 1));
    for (int r = 0; r < R; r++) {
      wr32(out + BLOB_HDR + 4 * r, (uint32_t)woff);
      lay_out_row(rows[r], slen + (size_t)r * C, C, laid);
      memcpy(out + geo.off_pay + 4 * woff, laid, 4 * (size_t)rowlen[r]);
      woff += rowlen[r];
    }
    free(laid);
    if (!coded) memcpy(out + geo.off_anchor, anchors, 2 * (size_t)L * ng * C);
    memcpy(out + geo.off_len, slen, 2 * (size_t)R * C);
    *len = total;
  }
  for (int r = 0; r < R; r++) free(rows[r]);
  free(rows); free(rowlen); free(slen); free(anchors);
  return rc;
}

int cgo_chunk_symbols(const uint8_t* tables, size_t tlen, const uint16_t* k,
                      const uint16_t* v, int chunk, int q, int8_t* anchors,
                      uint8_t* syms) {
  tabview tv;
  int32_t t0, tc, ng;
  if (parse_tables(tables, tlen, &tv) != OK) return E_INVAL;
  if (q < 0 || q > 2 || !tv.freq[q]) return E_MISMATCH;
  if (cgo_chunk_geometry(tables, tlen, chunk, &t0, &tc, &ng) != OK) return E_INVAL;
  const int L = tv.p.layers, C = tv.p.channels, T = tv.p.tokens, G = tv.p.group_tokens;
  const size_t lc = (size_t)L * C;
  int8_t* anc = (int8_t*)malloc(ng);
  uint8_t* pt = (uint8_t*)malloc(tc);
  for (int kv = 0; kv < 2; kv++)
    for (int l = 0; l < L; l++)
      for (int c = 0; c < C; c++) {
        size_t i = kv * lc + (size_t)l * C + c;
        const uint16_t* x = (kv ? v : k) + ((size_t)l * T + t0) * C + c;
        channel_symbols(x, C, tc, G, tv_f(tv.scale_a, i), tv_f(tv.inv_a, i),
                        tv_f(tv.inv_step[q], i), anc, NULL, pt);
        for (int g = 0; g < ng; g++) anchors[(((size_t)kv * L + l) * ng + g) * C + c] = anc[g];
        for (int t = 0; t < tc; t++) syms[(((size_t)kv * L + l) * tc + t) * C + c] = pt[t];
      }
  free(anc);
  free(pt);
  return OK;
}

/* parsed view of a blob, checked against the tables */
typedef struct {
  int32_t L, C, T, t0, tc, G, ng, q;
  uint32_t W;
  uint64_t id;
  int coded;               /* anchors range-coded (version 3) */
  const uint8_t* rows;     /* u32 [rows]: [2][L] delta rows, then [2][L] anchor rows if coded */
  const int8_t* anchors;   /* i8 [2][L][ng][C], raw anchors only */
  const uint8_t* lens;     /* u16 [rows][C] */
  const uint8_t* payload;  /* W big-endian-within-word u32 words */
  size_t payload_bytes_avail; /* payload plus trailing padding */
} blobview;

static int parse_blob(const tabview* tv, const uint8_t* b, size_t blen, blobview* bv) {
  if (blen < BLOB_HDR || rd32(b) != BLOB_MAGIC) return E_INVAL;
  uint32_t version = rd32(b + 4);
  if (version != BLOB_VERSION && version != BLOB_VERSION_CODED) return E_INVAL;
  bv->coded = version == BLOB_VERSION_CODED;
  bv->L = rdi32(b + 8); bv->C = rdi32(b + 12); bv->T = rdi32(b + 16);
  bv->t0 = rdi32(b + 20); bv->tc = rdi32(b + 24); bv->G = rdi32(b + 28);
  bv->ng = rdi32(b + 32); bv->q = rdi32(b + 36); bv->W = rd32(b + 40);
  bv->id = rd64(b + 48);
  if (rd32(b + 44) != PBITS) return E_INVAL;
  if (bv->L != tv->p.layers || bv->C != tv->p.channels || bv->T != tv->p.tokens ||
      bv->G != tv->p.group_tokens)
    return E_MISMATCH;
  if (bv->id != tv->id) return E_MISMATCH;
  if (bv->coded != (tv->afreq != NULL)) return E_MISMATCH;
  if (bv->q < 0 || bv->q > 2 || !tv->freq[bv->q]) return E_MISMATCH;
  int CH = tv->p.chunk_tokens;
  if (bv->t0 < 0 || bv->t0 % CH || bv->t0 >= bv->T) return E_INVAL;
  int tc = (bv->T - bv->t0 < CH) ? bv->T - bv->t0 : CH;
  if (bv->tc != tc || bv->ng != (tc + bv->G - 1) / bv->G) return E_INVAL;
  const blobgeo geo = blob_geometry(bv->L, bv->C, bv->ng, bv->coded);
  if (align16(geo.off_pay + 4 * (size_t)bv->W + 16) > blen) return E_INVAL;
  bv->rows = b + BLOB_HDR;
  bv->anchors = bv->coded ? NULL : (const int8_t*)(b + geo.off_anchor);
  bv->lens = b + geo.off_len;
  bv->payload = b + geo.off_pay;
  bv->payload_bytes_avail = blen - geo.off_pay;
  return OK;
}

/* The byte string of stream j of the block at payload word `base` (each word
 * holds four stream bytes, most significant first), read through the payload
 * layout; words outside the payload read as zero.  Whatever follows a stream
 * does not change what it decodes to (its flush names a block inside the
 * final interval), so the decoder reads on into zeros. */
static uint8_t* stream_bytes(const blobview* bv, size_t base, int ns, int m, const size_t* tail,
                             int j, size_t len, size_t* nb) {
  size_t words = bv->payload_bytes_avail / 4;
  uint8_t* out = (uint8_t*)malloc(4 * len + 1);
  for (size_t w = 0; w < len; w++) {
    size_t at = base + block_word(ns, m, tail, j, w);
    uint32_t v = at < words ? rd32(bv->payload + 4 * at) : 0;
    out[4 * w] = (uint8_t)(v >> 24);
    out[4 * w + 1] = (uint8_t)(v >> 16);
    out[4 * w + 2] = (uint8_t)(v >> 8);
    out[4 * w + 3] = (uint8_t)v;
  }
  *nb = 4 * len;
  return out;
}

/* The streams of payload row r, channel after channel: each stream starts at
 * the row offset plus the lengths of the streams before it, laid out by
 * blocks as in lay_out_row. */
typedef struct {
  const blobview* bv;
  int r, R, C, ns, m;
  size_t w, bbase;
  uint16_t blen16[BLOCK_STREAMS];
  size_t tail[BLOCK_STREAMS];
} rowwalk;

static void rowwalk_start(rowwalk* it, const blobview* bv, int r, int R, int C) {
  it->bv = bv;
  it->r = r;
  it->R = R;
  it->C = C;
  it->w = rd32(bv->rows + 4 * (size_t)r);
  it->bbase = it->w;
  it->ns = it->m = 0;
}

/* bytes of stream c of the row (called for c = 0, 1, ... in order); sets
 * *over when the stream runs past the payload */
static uint8_t* rowwalk_next(rowwalk* it, int c, size_t* nb, int* over) {
  const blobview* bv = it->bv;
  if (c % BLOCK_STREAMS == 0) { /* a new block: its streams' lengths and layout */
    size_t i = (size_t)it->r * it->C + c;
    it->bbase = it->w;
    it->ns = it->C - c < BLOCK_STREAMS ? it->C - c : BLOCK_STREAMS;
    for (int j = 0; j < it->ns; j++)
      it->blen16[j] = (uint16_t)(bv->lens[2 * (i + j)] | (bv->lens[2 * (i + j) + 1] << 8));
    it->m = block_units(it->blen16, it->ns);
    block_tails(it->blen16, it->ns, it->m, it->tail);
  }
  size_t slw = it->blen16[c % BLOCK_STREAMS];
  if (it->w + slw > bv->W) *over = 1;
  uint8_t* bytes = stream_bytes(bv, it->bbase, it->ns, it->m, it->tail, c % BLOCK_STREAMS, slw, nb);
  it->w += slw;
  return bytes;
}

/* whether the row's streams end where the next row starts */
static int rowwalk_ends_right(const rowwalk* it) {
  size_t next = (it->r + 1 < it->R) ? rd32(it->bv->rows + 4 * (size_t)(it->r + 1)) : it->bv->W;
  return it->w == next;
}

/* decode a blob's rows: for coded anchors the (kv, layer) row's anchor streams
 * first, then its delta streams; the decoder reads on into whatever bytes
 * follow a stream */
static int decode_blob_impl(const uint8_t* tables, size_t tlen, const uint8_t* blob,
                            size_t blen, uint16_t* k_out, uint16_t* v_out, uint8_t* syms,
                            int nthreads, int* corrupt) {
  tabview tv;
  blobview bv;
  *corrupt = 0;
  if (parse_tables(tables, tlen, &tv) != OK) return E_INVAL;
  int rc = parse_blob(&tv, blob, blen, &bv);
  if (rc != OK) return rc;
  if (nthreads <= 0) nthreads = 1;
  const int L = bv.L, C = bv.C, T = bv.T, G = bv.G, tc = bv.tc, ng = bv.ng, q = bv.q;
  const int R = bv.coded ? 4 * L : 2 * L;
  const size_t lc = (size_t)L * C;
  const int nsyms = tc - ng;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
  for (int row = 0; row < 2 * L; row++) {
    int kv = row / L, l = row % L;
    uint8_t* sym = (uint8_t*)malloc((nsyms > ng ? nsyms : ng) + 1);
    /* the row's anchors [ng][C] */
    int8_t* anc = (int8_t*)malloc((size_t)ng * C + 1);
    rowwalk it;
    size_t nb = 0;
    if (bv.coded) {
      uint16_t af[ASYM];
      memcpy(af, tv.afreq + 2 * ASYM * ((size_t)kv * L + l), sizeof(af));
      rowwalk_start(&it, &bv, 2 * L + row, R, C);
      for (int c = 0; c < C; c++) {
        int cor = 0;
        uint8_t* bytes = rowwalk_next(&it, c, &nb, &cor);
        if (cgo_rc_decode(bytes, nb, ng, af, ASYM, sym, NULL, &cor) != OK) {
          cor = 1; /* an unusable anchor table */
          memset(sym, 128, ng);
        }
        free(bytes);
        if (cor) bad = 1;
        for (int g = 0; g < ng; g++) anc[(size_t)g * C + c] = (int8_t)(sym[g] - 128);
      }
      if (!rowwalk_ends_right(&it)) bad = 1; /* lengths disagree with the row offsets */
    } else {
      memcpy(anc, bv.anchors + ((size_t)kv * L + l) * ng * C, (size_t)ng * C);
    }
    rowwalk_start(&it, &bv, row, R, C);
    for (int c = 0; c < C; c++) {
      size_t i = kv * lc + (size_t)l * C + c;
      int cor = 0;
      uint8_t* bytes = rowwalk_next(&it, c, &nb, &cor);
      uint16_t f[NSYM];
      tv_freq(tv.freq[q], i, f);
      if (cgo_rc_decode(bytes, nb, nsyms, f, NSYM, sym, NULL, &cor) != OK) {
        cor = 1; /* an unusable frequency table: the stream is corrupt */
        memset(sym, 32, nsyms);
      }
      free(bytes);
      if (cor) bad = 1;
      float scale_a = tv_f(tv.scale_a, i), step = tv_f(tv.step[q], i);
      int ns = 0, g = 0;
      for (int g0 = 0; g0 < tc; g0 += G, g++) {
        int ge = (g0 + G < tc) ? g0 + G : tc;
        int8_t a = anc[(size_t)g * C + c];
        float ahat = anchor_value(a, scale_a);
        size_t o = ((size_t)l * T + bv.t0 + g0) * C + c;
        if (k_out) (kv ? v_out : k_out)[o] = cgo_f32_to_f16(ahat);
        if (syms) syms[(((size_t)kv * L + l) * tc + g0) * C + c] = 255;
        for (int t = g0 + 1; t < ge; t++) {
          uint8_t s = sym[ns++];
          size_t ot = ((size_t)l * T + bv.t0 + t) * C + c;
          if (k_out) (kv ? v_out : k_out)[ot] = dequant_delta(s, step, ahat);
          if (syms) syms[(((size_t)kv * L + l) * tc + t) * C + c] = s;
        }
      }
    }
    if (!rowwalk_ends_right(&it)) bad = 1; /* lengths disagree with the row offsets */
    free(sym);
    free(anc);
  }
  *corrupt = bad;
  return OK;
}

int cgo_decode_blob(const uint8_t* tables, size_t tlen, const uint8_t* blob, size_t blen,
                    uint16_t* k_out, uint16_t* v_out, int nthreads, int* corrupt) {
  return decode_blob_impl(tables, tlen, blob, blen, k_out, v_out, NULL, nthreads, corrupt);
}

int cgo_decode_blob_symbols(const uint8_t* tables, size_t tlen, const uint8_t* blob,
                            size_t blen, uint8_t* syms, int* corrupt) {
  return decode_blob_impl(tables, tlen, blob, blen, NULL, NULL, syms, 1, corrupt);
}

/* ------------------------------------------------------------------------- */
/* Single streams                                                             */
/* ------------------------------------------------------------------------- */

int cgo_stream_encode(const uint8_t* tables, size_t tlen, int kv, int l, int c, int q,
                      const uint16_t* x, int tc, int8_t* anchors, uint8_t* out,
                      size_t cap, size_t* len) {
  tabview tv;
  if (parse_tables(tables, tlen, &tv) != OK) return E_INVAL;
  if (q < 0 || q > 2 || !tv.freq[q]) return E_MISMATCH;
  if (kv < 0 || kv > 1 || l < 0 || l >= tv.p.layers || c < 0 || c >= tv.p.channels ||
      tc < 1 || tc > tv.p.chunk_tokens)
    return E_INVAL;
  const int G = tv.p.group_tokens, ng = (tc + G - 1) / G;
  size_t i = (size_t)kv * tv.p.layers * tv.p.channels + (size_t)l * tv.p.channels + c;
  if (any_nonfinite(x, 1, tc)) return E_INVAL;
  uint8_t* sym = (uint8_t*)malloc(tc);
  channel_symbols(x, 1, tc, G, tv_f(tv.scale_a, i), tv_f(tv.inv_a, i),
                  tv_f(tv.inv_step[q], i), anchors, sym, NULL);
  uint16_t f[NSYM];
  tv_freq(tv.freq[q], i, f);
  size_t nb = 0, bound = cgo_rc_bound(tc - ng);
  uint8_t* bytes = (uint8_t*)malloc(bound + 1);
  int rc = cgo_rc_encode(sym, tc - ng, f, NSYM, bytes, bound + 1, &nb);
  free(sym);
  if (rc == OK) {
    size_t padded = (nb + 3) & ~(size_t)3;
    if (padded > cap) {
      rc = E_CAPACITY;
    } else {
      memset(out, 0, padded);
      memcpy(out, bytes, nb);
      *len = padded;
    }
  }
  free(bytes);
  return rc;
}

int cgo_stream_decode(const uint8_t* tables, size_t tlen, int kv, int l, int c, int q,
                      const int8_t* anchors, int tc, const uint8_t* bytes,
                      size_t nbytes, uint16_t* y, int* corrupt) {
  tabview tv;
  if (parse_tables(tables, tlen, &tv) != OK) return E_INVAL;
  if (q < 0 || q > 2 || !tv.freq[q]) return E_MISMATCH;
  if (kv < 0 || kv > 1 || l < 0 || l >= tv.p.layers || c < 0 || c >= tv.p.channels ||
      tc < 1 || tc > tv.p.chunk_tokens)
    return E_INVAL;
  const int G = tv.p.group_tokens, ng = (tc + G - 1) / G;
  size_t i = (size_t)kv * tv.p.layers * tv.p.channels + (size_t)l * tv.p.channels + c;
  uint8_t* sym = (uint8_t*)malloc(tc);
  uint16_t f[NSYM];
  tv_freq(tv.freq[q], i, f);
  *corrupt = 0;
  if (cgo_rc_decode(bytes, nbytes, tc - ng, f, NSYM, sym, NULL, corrupt) != OK) {
    *corrupt = 1; /* an unusable frequency table */
    memset(sym, 32, tc);
  }
  float scale_a = tv_f(tv.scale_a, i), step = tv_f(tv.step[q], i);
  int ns = 0, g = 0;
  for (int g0 = 0; g0 < tc; g0 += G, g++) {
    int ge = (g0 + G < tc) ? g0 + G : tc;
    float ahat = anchor_value(anchors[g], scale_a);
    y[g0] = cgo_f32_to_f16(ahat);
    for (int t = g0 + 1; t < ge; t++) y[t] = dequant_delta(sym[ns++], step, ahat);
  }
  free(sym);
  return OK;
}
