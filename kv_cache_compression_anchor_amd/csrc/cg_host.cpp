// Host-side checks of libcachegen's C ABI: parameters, chunk blob headers,
// serialized table images, the per-chunk quality choice and the error
// message of the calling thread.  No HIP here: every check also builds on its
// own, under the CPU sanitizers.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <string>

#include "cg_format.h"

namespace cg {

namespace {
thread_local std::string g_err;
}  // namespace

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

// n_layer_groups = 0 asks for the default split: the pages' three groups of a
// 32-layer model (layers 1-10, 11-20, 21-32) scaled to L layers, ends
// floor(10 L / 32), floor(20 L / 32), L.  The caller's params with that split
// filled in, or CG_E_INVAL when L is too small for three non-empty groups.
int resolve_params(const cg_params* in, cg_params* out) {
  if (!in) return fail(CG_E_INVAL, "params is NULL");
  *out = *in;
  if (in->n_layer_groups != 0) return CG_OK;
  if (in->layers < 4)
    return fail(CG_E_INVAL, "the default layer groups (n_layer_groups = 0) need at least 4 layers");
  out->n_layer_groups = 3;
  out->layer_group_end[0] = (int32_t)((int64_t)in->layers * 10 / 32);
  out->layer_group_end[1] = (int32_t)((int64_t)in->layers * 20 / 32);
  out->layer_group_end[2] = in->layers;
  return CG_OK;
}

int check_params(const cg_params* p) {
  if (!p) return fail(CG_E_INVAL, "params is NULL");
  if (p->layers < 1 || p->tokens < 1 || p->channels < 1)
    return fail(CG_E_INVAL, "layers, tokens and channels must be positive");
  if (p->layers > 4096 || p->channels > 65536 || p->tokens > kMaxTokens)
    return fail(CG_E_INVAL, "shape too large (layers <= 4096, channels <= 65536, tokens <= 2^21)");
  if (p->chunk_tokens < 1 || p->chunk_tokens > kMaxChunk)
    return fail(CG_E_INVAL, "chunk_tokens must be in 1..65536");
  if (p->group_tokens < 1 || p->group_tokens > p->chunk_tokens)
    return fail(CG_E_INVAL, "group_tokens must be in 1..chunk_tokens");
  // one chunk of one (kv, layer) row is addressed through 32-bit buffer ranges
  // and row offsets (token row x 2 C bytes): it must stay below 4 GiB
  if ((uint64_t)std::min(p->chunk_tokens, p->tokens) * (uint64_t)p->channels * 2u >= (1ull << 32))
    return fail(CG_E_INVAL, "a chunk of one layer (chunk_tokens x channels x 2 bytes) must be "
                            "smaller than 4 GiB");
  if (p->n_layer_groups < 1 || p->n_layer_groups > 3)
    return fail(CG_E_INVAL, "n_layer_groups must be 1..3");
  int prev = 0;
  for (int i = 0; i < p->n_layer_groups; i++) {
    if (p->layer_group_end[i] <= prev) return fail(CG_E_INVAL, "layer_group_end must increase");
    prev = p->layer_group_end[i];
    if (!(p->layer_step[i] > 0.0f) || !isfinite(p->layer_step[i]))
      return fail(CG_E_INVAL, "layer_step must be positive and finite");
  }
  if (prev != p->layers) return fail(CG_E_INVAL, "last layer_group_end must equal layers");
  if ((p->quality_mask & ~7u) || !p->quality_mask)
    return fail(CG_E_INVAL, "quality_mask must be a non-empty subset of {H,M,L}");
  if (p->anchor_coding != 0 && p->anchor_coding != 1)
    return fail(CG_E_INVAL, "anchor_coding must be 0 or 1");
  // an anchor table counts the channels x groups of a layer in 32 bits
  if (p->anchor_coding && (uint64_t)p->channels * (uint64_t)p->tokens >= (1ull << 32))
    return fail(CG_E_INVAL, "coded anchors need channels x tokens below 2^32");
  for (int q = 0; q < 3; q++)
    if ((p->quality_mask >> q) & 1)
      if (!(p->quality_mult[q] > 0.0f) || !isfinite(p->quality_mult[q]))
        return fail(CG_E_INVAL, "quality_mult must be positive and finite");
  const size_t n = (size_t)2 * p->layers * p->channels;
  const TabLayout lay = tab_layout(p->layers, p->channels, p->quality_mask, p->anchor_coding != 0);
  if (lay.total > 0x7FFFFFFFull || n > 0x7FFFFFFFull)
    return fail(CG_E_INVAL, "tables larger than 2 GiB");
  return CG_OK;
}

int parse_info(const uint8_t* b, size_t len, cg_chunk_info* o) {
  if (!b || !o) return fail(CG_E_INVAL, "NULL argument");
  if (len < (size_t)kBlobHdr) return fail(CG_E_INVAL, "blob shorter than its header");
  uint32_t u[16];
  memcpy(u, b, 64);
  if (u[0] != kBlobMagic || (u[1] != kBlobVersion && u[1] != kBlobVersionCoded))
    return fail(CG_E_INVAL, "not a CGK1 version 2 or 3 blob");
  if (u[11] != (uint32_t)kProbBits) return fail(CG_E_INVAL, "unsupported probability precision");
  o->layers = (int32_t)u[2];
  o->channels = (int32_t)u[3];
  o->total_tokens = (int32_t)u[4];
  o->token_offset = (int32_t)u[5];
  o->chunk_tokens = (int32_t)u[6];
  o->group_tokens = (int32_t)u[7];
  o->n_groups = (int32_t)u[8];
  o->quality = (int32_t)u[9];
  o->payload_words = u[10];
  o->version = u[1];
  memcpy(&o->tables_id, &u[12], 8);
  if (o->layers < 1 || o->layers > 4096 || o->channels < 1 || o->channels > 65536 ||
      o->total_tokens < 1 || o->total_tokens > kMaxTokens || o->chunk_tokens < 1 ||
      o->chunk_tokens > kMaxChunk || o->group_tokens < 1 || o->token_offset < 0 ||
      o->token_offset >= o->total_tokens ||
      o->chunk_tokens > o->total_tokens - o->token_offset || o->quality < 0 || o->quality > 2 ||
      o->n_groups != (o->chunk_tokens + o->group_tokens - 1) / o->group_tokens ||
      o->payload_words > 0x3FFFFFFFu)
    return fail(CG_E_INVAL, "inconsistent blob header");
  if ((uint64_t)o->chunk_tokens * (uint64_t)o->channels * 2u >= (1ull << 32))
    return fail(CG_E_INVAL, "a chunk of one layer (chunk_tokens x channels x 2 bytes) must be "
                            "smaller than 4 GiB");
  const BlobLayout bl = blob_layout(o->layers, o->channels, o->n_groups, o->version == kBlobVersionCoded);
  o->blob_bytes = blob_bytes(bl, o->payload_words);
  if (o->blob_bytes > 0xFFFFFFFFull) return fail(CG_E_INVAL, "blob larger than 4 GiB");
  return CG_OK;
}

int check_tables_image(const uint8_t* b, size_t len, cg_params* out) {
  if (!b || !out) return fail(CG_E_INVAL, "NULL argument");
  if (len < (size_t)kTabHdr) return fail(CG_E_INVAL, "tables shorter than their header");
  uint32_t u[20];
  memcpy(u, b, kTabHdr);
  if (u[0] != kTabMagic || (u[1] != kTabVersion && u[1] != kTabVersionCoded) ||
      u[18] != (uint32_t)kProbBits || u[19] != (uint32_t)kNSym)
    return fail(CG_E_INVAL, "not CGT1 version 1 or 2 tables");
  cg_params p;
  memset(&p, 0, sizeof(p));
  p.layers = (int32_t)u[2];
  p.channels = (int32_t)u[3];
  p.tokens = (int32_t)u[4];
  p.chunk_tokens = (int32_t)u[5];
  p.group_tokens = (int32_t)u[6];
  p.n_layer_groups = (int32_t)u[7];
  for (int i = 0; i < 3; i++) {
    p.layer_group_end[i] = (int32_t)u[8 + i];
    memcpy(&p.layer_step[i], &u[11 + i], 4);
    memcpy(&p.quality_mult[i], &u[14 + i], 4);
  }
  p.quality_mask = u[17];
  p.anchor_coding = u[1] == kTabVersionCoded ? 1 : 0;
  const int rc = check_params(&p);
  if (rc) return rc;
  const TabLayout lay = tab_layout(p.layers, p.channels, p.quality_mask, p.anchor_coding != 0);
  if (len != lay.total) return fail(CG_E_INVAL, "tables size does not match their header");
  // every value the kernels rely on: positive normal steps, finite inverses,
  // frequency tables of 64 positive entries summing to 2^15
  for (size_t i = 0; i < lay.n; i++) {
    float sa, ia;
    memcpy(&sa, b + lay.off_scale_a + 4 * i, 4);
    memcpy(&ia, b + lay.off_inv_a + 4 * i, 4);
    if (!(sa > 0.0f) || !isfinite(sa) || !isfinite(ia)) return fail(CG_E_INVAL, "bad anchor scale");
  }
  for (int q = 0; q < 3; q++) {
    if (!((p.quality_mask >> q) & 1)) continue;
    for (size_t i = 0; i < lay.n; i++) {
      float s, is;
      memcpy(&s, b + lay.off_step[q] + 4 * i, 4);
      memcpy(&is, b + lay.off_inv_step[q] + 4 * i, 4);
      if (!(s >= 1.17549435e-38f) || !isfinite(s) || !isfinite(is))
        return fail(CG_E_INVAL, "bad delta step");
      uint16_t f[kNSym];
      memcpy(f, b + lay.off_freq[q] + 2 * kNSym * i, sizeof(f));
      uint32_t sum = 0;
      for (int k = 0; k < kNSym; k++) {
        if (!f[k]) return fail(CG_E_INVAL, "zero frequency");
        sum += f[k];
      }
      if (sum != kProbTotal) return fail(CG_E_INVAL, "frequencies do not sum to 2^15");
    }
  }
  if (lay.off_afreq) {
    for (size_t i = 0; i < (size_t)2 * p.layers; i++) {
      uint16_t f[kASym];
      memcpy(f, b + lay.off_afreq + 2 * kASym * i, sizeof(f));
      uint32_t sum = 0;
      for (int k = 0; k < kASym; k++) {
        if (!f[k]) return fail(CG_E_INVAL, "zero anchor frequency");
        sum += f[k];
      }
      if (sum != kProbTotal) return fail(CG_E_INVAL, "anchor frequencies do not sum to 2^15");
    }
  }
  *out = p;
  return CG_OK;
}

}  // namespace cg

using namespace cg;

extern "C" {

const char* cg_last_error(void) { return g_err.c_str(); }

int cg_plan_chunk(const cg_chunk_plan_in* in, int32_t* quality_out, double* ratio_out) {
  if (!in || !quality_out) return fail(CG_E_INVAL, "NULL argument");
  if (!(in->bandwidth_bpms > 0.0) || !std::isfinite(in->bandwidth_bpms))
    return fail(CG_E_INVAL, "bandwidth must be positive and finite");
  if (std::isnan(in->budget_ms)) return fail(CG_E_INVAL, "budget is NaN");
  double r[3] = {0.0, 0.0, 0.0};
  double best_end = 0.0;
  int best = -1, first_fit = -1;
  for (int q = 0; q < 3; q++) {
    const double d = in->decode_ms_left[q];
    if (!(d >= 0.0) || !std::isfinite(d)) return fail(CG_E_INVAL, "bad decode time");
    if (in->bytes_left[q] == 0) continue;
    const double t_send = (double)in->bytes_left[q] / in->bandwidth_bpms;
    r[q] = (in->budget_ms - d) / t_send;
    if (first_fit < 0 && r[q] >= 1.0) first_fit = q;
    const double end = t_send + d;  // when nothing fits: the version done soonest
    if (best < 0 || end < best_end) {
      best = q;
      best_end = end;
    }
  }
  if (best < 0) return fail(CG_E_INVAL, "no version of the chunk");
  *quality_out = first_fit >= 0 ? first_fit : best;
  if (ratio_out)
    for (int q = 0; q < 3; q++) ratio_out[q] = r[q];
  return CG_OK;
}

int cg_chunk_info_parse(const void* blob_host, size_t len, cg_chunk_info* out) {
  return parse_info(static_cast<const uint8_t*>(blob_host), len, out);
}

}  // extern "C"
