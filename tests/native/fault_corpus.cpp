// Fault corpus for the host-side checks of libcachegen (cg_host.cpp: parameter
// checks, blob header parsing, table image checks, the per-chunk quality
// choice) and for the CPU oracle's table and blob parsing and decoding.  Built
// and run on the CPU under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitize.py: every malformed input must come back as an error (or,
// for the oracle's decoder on damaged stream bytes, as a decode flagged
// corrupt), never as a crash, an out-of-bounds access or undefined behaviour.
//
// Inputs: a small valid table image and blob written by the oracle from seeded
// synthetic K/V, then truncated, bit-flipped, overwritten field by field and
// resized.  Prints "fault corpus ok: N cases" and exits 0 when every
// expectation holds.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "cachegen.h"
#include "cg_format.h"
#include "cgoracle.h"

namespace {

int g_cases = 0, g_failures = 0;

void expect(bool ok, const std::string& what) {
  g_cases++;
  if (!ok) {
    g_failures++;
    fprintf(stderr, "FAIL: %s\n", what.c_str());
  }
}

// xorshift64*: the corpus' only source of randomness
struct Rng {
  uint64_t s;
  uint64_t next() {
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    return s * 2685821657736338717ull;
  }
  double uniform() { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }
  size_t below(size_t n) { return (size_t)(next() % n); }
};

// small workload: a ragged 64-channel block, three chunks (the last short), a
// last group of the chunk shorter than the others
constexpr int L = 2, T = 50, C = 70, CH = 24, G = 5;

cgo_params oracle_params(int anchor_coding) {
  cgo_params p;
  memset(&p, 0, sizeof(p));
  p.layers = L;
  p.tokens = T;
  p.channels = C;
  p.chunk_tokens = CH;
  p.group_tokens = G;
  p.n_layer_groups = 2;
  p.layer_group_end[0] = 1;
  p.layer_group_end[1] = 2;
  p.layer_step[0] = 0.5f;
  p.layer_step[1] = 1.0f;
  p.quality_mult[0] = 1.0f;
  p.quality_mult[1] = 2.0f;
  p.quality_mult[2] = 4.0f;
  p.quality_mask = 7;
  p.anchor_coding = anchor_coding;
  return p;
}

cg_params lib_params() {
  const cgo_params o = oracle_params(0);
  cg_params p;
  memset(&p, 0, sizeof(p));
  p.layers = o.layers;
  p.tokens = o.tokens;
  p.channels = o.channels;
  p.chunk_tokens = o.chunk_tokens;
  p.group_tokens = o.group_tokens;
  p.n_layer_groups = o.n_layer_groups;
  for (int i = 0; i < 3; i++) {
    p.layer_group_end[i] = o.layer_group_end[i];
    p.layer_step[i] = o.layer_step[i];
    p.quality_mult[i] = o.quality_mult[i];
  }
  p.quality_mask = o.quality_mask;
  return p;
}

// AR(1) K/V rows with per-channel scales, as binary16
void make_kv(std::vector<uint16_t>& k, std::vector<uint16_t>& v) {
  Rng r{0x9E3779B97F4A7C15ull};
  k.resize((size_t)L * T * C);
  v.resize(k.size());
  for (int which = 0; which < 2; which++) {
    std::vector<uint16_t>& x = which ? v : k;
    for (int l = 0; l < L; l++)
      for (int c = 0; c < C; c++) {
        const double scale = 0.05 + 2.0 * r.uniform();
        double s = 0.0;
        for (int t = 0; t < T; t++) {
          const double g = (r.uniform() + r.uniform() + r.uniform() - 1.5) * 2.0;
          s = 0.9 * s + 0.44 * g;
          x[((size_t)l * T + t) * C + c] = cgo_f32_to_f16((float)(s * scale));
        }
      }
  }
}

int oracle_decode(const std::vector<uint8_t>& tab, const uint8_t* blob, size_t blen, int* corrupt) {
  std::vector<uint16_t> ko((size_t)L * T * C), vo(ko.size());
  *corrupt = 0;
  return cgo_decode_blob(tab.data(), tab.size(), blob, blen, ko.data(), vo.data(), 1, corrupt);
}

void put32(std::vector<uint8_t>& b, size_t off, uint32_t x) { memcpy(b.data() + off, &x, 4); }

void params_cases() {
  const cg_params good = lib_params();
  expect(cg::check_params(&good) == CG_OK, "valid params accepted");
  expect(cg::check_params(nullptr) == CG_E_INVAL, "NULL params rejected");
  struct Bad {
    const char* what;
    void (*edit)(cg_params&);
  };
  const Bad bad[] = {
      {"zero layers", [](cg_params& p) { p.layers = 0; }},
      {"negative tokens", [](cg_params& p) { p.tokens = -5; }},
      {"too many channels", [](cg_params& p) { p.channels = 65537; }},
      {"chunk of zero tokens", [](cg_params& p) { p.chunk_tokens = 0; }},
      {"group longer than the chunk", [](cg_params& p) { p.group_tokens = p.chunk_tokens + 1; }},
      {"chunk of 4 GiB per layer",
       [](cg_params& p) { p.tokens = 65536; p.chunk_tokens = 65536; p.channels = 32768; }},
      {"four layer groups", [](cg_params& p) { p.n_layer_groups = 4; }},
      {"layer groups not increasing", [](cg_params& p) { p.layer_group_end[1] = 1; }},
      {"last group not the last layer", [](cg_params& p) { p.layer_group_end[1] = 3; }},
      {"NaN step", [](cg_params& p) { p.layer_step[0] = NAN; }},
      {"infinite step", [](cg_params& p) { p.layer_step[1] = INFINITY; }},
      {"zero step", [](cg_params& p) { p.layer_step[0] = 0.0f; }},
      {"empty quality mask", [](cg_params& p) { p.quality_mask = 0; }},
      {"unknown quality", [](cg_params& p) { p.quality_mask = 9; }},
      {"negative quality multiplier", [](cg_params& p) { p.quality_mult[2] = -1.0f; }},
  };
  for (const Bad& b : bad) {
    cg_params p = good;
    b.edit(p);
    expect(cg::check_params(&p) == CG_E_INVAL, std::string("params: ") + b.what);
    expect(strlen(cg_last_error()) > 0, std::string("error message for ") + b.what);
  }
  cg_params d = good;
  d.n_layer_groups = 0;
  cg_params out;
  expect(cg::resolve_params(&d, &out) == CG_E_INVAL, "default layer groups need 4 layers");
  d.layers = 32;
  d.layer_step[2] = 1.5f;
  expect(cg::resolve_params(&d, &out) == CG_OK && out.n_layer_groups == 3 &&
             out.layer_group_end[0] == 10 && out.layer_group_end[1] == 20 &&
             out.layer_group_end[2] == 32 && cg::check_params(&out) == CG_OK,
         "default layer groups of a 32-layer model");
  expect(cg::resolve_params(nullptr, &out) == CG_E_INVAL, "NULL params to resolve");
}

void plan_cases() {
  cg_chunk_plan_in in;
  memset(&in, 0, sizeof(in));
  in.bandwidth_bpms = 1e6;
  in.budget_ms = 10.0;
  for (int q = 0; q < 3; q++) {
    in.bytes_left[q] = (uint64_t)(1000000 >> q);
    in.decode_ms_left[q] = 0.5;
  }
  int32_t q = -1;
  double ratio[3];
  expect(cg_plan_chunk(&in, &q, ratio) == CG_OK && q >= 0 && q <= 2, "valid plan");
  const double bad_bw[] = {0.0, -1.0, NAN, INFINITY};
  for (double b : bad_bw) {
    cg_chunk_plan_in x = in;
    x.bandwidth_bpms = b;
    expect(cg_plan_chunk(&x, &q, ratio) == CG_E_INVAL, "plan: bad bandwidth");
  }
  cg_chunk_plan_in x = in;
  x.budget_ms = NAN;
  expect(cg_plan_chunk(&x, &q, ratio) == CG_E_INVAL, "plan: NaN budget");
  x = in;
  x.decode_ms_left[1] = -1.0;
  expect(cg_plan_chunk(&x, &q, ratio) == CG_E_INVAL, "plan: negative decode time");
  x = in;
  for (int k = 0; k < 3; k++) x.bytes_left[k] = 0;
  expect(cg_plan_chunk(&x, &q, ratio) == CG_E_INVAL, "plan: no version left");
  expect(cg_plan_chunk(nullptr, &q, ratio) == CG_E_INVAL, "plan: NULL input");
  expect(cg_plan_chunk(&in, nullptr, ratio) == CG_E_INVAL, "plan: NULL output");
}

void table_cases(const std::vector<uint8_t>& tab, const uint8_t* blob, size_t blen, bool coded) {
  cg_params p;
  expect(cg::check_tables_image(tab.data(), tab.size(), &p) == CG_OK, "valid table image");
  expect(p.layers == L && p.channels == C && p.tokens == T && p.anchor_coding == (int)coded,
         "table image params");
  int32_t t0, tc, ng;
  expect(cgo_chunk_geometry(tab.data(), tab.size(), 2, &t0, &tc, &ng) == 0 && tc == T - 2 * CH,
         "oracle geometry of the short chunk");
  expect(cgo_chunk_geometry(tab.data(), tab.size(), 3, &t0, &tc, &ng) != 0,
         "oracle geometry past the last chunk");

  // truncations: a copy of exactly that many bytes, so any over-read is caught
  const size_t cuts[] = {0, 1, 79, 80, 81, tab.size() / 2, tab.size() - 1};
  for (size_t n : cuts) {
    std::vector<uint8_t> t(tab.begin(), tab.begin() + n);
    expect(cg::check_tables_image(t.data(), n, &p) != CG_OK, "truncated table image rejected");
    expect(cgo_chunk_geometry(t.data(), n, 0, &t0, &tc, &ng) != 0, "oracle: truncated tables");
    int corrupt;
    expect(oracle_decode(t, blob, blen, &corrupt) != 0, "oracle decode with truncated tables");
  }
  std::vector<uint8_t> longer(tab);
  longer.push_back(0);
  expect(cg::check_tables_image(longer.data(), longer.size(), &p) != CG_OK, "oversized table image");

  // header fields: magic, version, shape, groups, steps, mask, precision, alphabet
  struct Field {
    size_t off;
    uint32_t value;
  };
  // version 1 <-> 2 changes the expected size: rejected too
  const Field fields[] = {{0, 0}, {4, coded ? 1u : 2u}, {4, 3}, {8, 0}, {12, 0xFFFFFFFFu}, {16, 0}, {20, 0},
                          {24, 1000}, {28, 0}, {28, 5}, {32, 0}, {36, 0}, {44, 0x7FC00000u},
                          {48, 0xFF800000u}, {68, 0}, {68, 8}, {72, 14}, {76, 63}};
  for (const Field& f : fields) {
    std::vector<uint8_t> t(tab);
    put32(t, f.off, f.value);
    expect(cg::check_tables_image(t.data(), t.size(), &p) != CG_OK,
           "table header field at " + std::to_string(f.off) + " rejected");
    int corrupt;
    expect(oracle_decode(t, blob, blen, &corrupt) != 0,
           "oracle rejects tables with header field at " + std::to_string(f.off));
  }

  // body values the kernels rely on: scales, steps, frequency tables
  const cg::TabLayout lay = cg::tab_layout(L, C, 7, coded);
  struct Body {
    size_t off;
    uint32_t value;
    const char* what;
  };
  const Body body[] = {
      {lay.off_scale_a + 4 * 3, 0u, "zero anchor scale"},
      {lay.off_scale_a + 4 * 5, 0x7F800000u, "infinite anchor scale"},
      {lay.off_inv_a + 4 * 7, 0x7FC00000u, "NaN inverse anchor scale"},
      {lay.off_step[1] + 4 * 11, 0x00000001u, "subnormal step"},
      {lay.off_inv_step[2] + 4 * 13, 0xFF800000u, "infinite inverse step"},
  };
  for (const Body& b : body) {
    std::vector<uint8_t> t(tab);
    put32(t, b.off, b.value);
    expect(cg::check_tables_image(t.data(), t.size(), &p) != CG_OK, b.what);
  }
  {
    std::vector<uint8_t> t(tab);
    const size_t f = lay.off_freq[0] + 2 * cg::kNSym * 17;
    const uint16_t z = 0, big = 40000;
    memcpy(t.data() + f + 2 * 5, &z, 2);
    expect(cg::check_tables_image(t.data(), t.size(), &p) != CG_OK, "zero frequency rejected");
    memcpy(t.data() + f + 2 * 5, &big, 2);
    expect(cg::check_tables_image(t.data(), t.size(), &p) != CG_OK, "frequencies off 2^15");
  }
  if (coded) {
    std::vector<uint8_t> t(tab);
    const size_t f = lay.off_afreq + 2 * cg::kASym * 3;
    const uint16_t z = 0, big = 40000;
    memcpy(t.data() + f + 2 * 200, &z, 2);
    expect(cg::check_tables_image(t.data(), t.size(), &p) != CG_OK, "zero anchor frequency rejected");
    memcpy(t.data() + f + 2 * 200, &big, 2);
    expect(cg::check_tables_image(t.data(), t.size(), &p) != CG_OK, "anchor frequencies off 2^15");
  }

  // random bit flips anywhere: either check gives an answer, neither faults
  Rng r{12345};
  for (int i = 0; i < 3000; i++) {
    std::vector<uint8_t> t(tab);
    const size_t at = r.below(t.size());
    t[at] ^= (uint8_t)(1u << r.below(8));
    (void)cg::check_tables_image(t.data(), t.size(), &p);
    int corrupt;
    (void)oracle_decode(t, blob, blen, &corrupt);
    g_cases++;
  }
}

// a frequency table that no longer sums to 2^15 reaches the oracle's decoder
// only through tables whose id the blob names: the blob's tables id is
// patched to the damaged tables' id (the blob is coded at quality M)
void unbalanced_frequency_case(const std::vector<uint8_t>& tab, const std::vector<uint8_t>& blob,
                               bool coded) {
  std::vector<uint8_t> t(tab);
  const cg::TabLayout lay = cg::tab_layout(L, C, 7, coded);
  const uint16_t z = 0;
  memcpy(t.data() + (coded ? lay.off_afreq + 2 * cg::kASym * 2 + 2 * 130
                           : lay.off_freq[1] + 2 * cg::kNSym * 3 + 2 * 10),
         &z, 2);
  std::vector<uint8_t> b(blob);
  const uint64_t id = cgo_tables_id(t.data(), t.size());
  memcpy(b.data() + 48, &id, 8);
  int corrupt = 0;
  const int rc = oracle_decode(t, b.data(), b.size(), &corrupt);
  expect(rc != 0 || corrupt, "oracle flags a stream whose table does not sum to 2^15");
}

void blob_cases(const std::vector<uint8_t>& tab, const std::vector<uint8_t>& blob, bool coded) {
  cg_chunk_info info;
  expect(cg_chunk_info_parse(blob.data(), blob.size(), &info) == CG_OK, "valid blob header");
  expect(info.blob_bytes == blob.size() && info.version == (coded ? 3u : 2u),
         "blob size and version from its header");
  int corrupt = 1;
  expect(oracle_decode(tab, blob.data(), blob.size(), &corrupt) == 0 && corrupt == 0,
         "oracle decodes the valid blob");
  expect(cg_chunk_info_parse(nullptr, 64, &info) == CG_E_INVAL, "NULL blob");
  expect(cg_chunk_info_parse(blob.data(), 64, nullptr) == CG_E_INVAL, "NULL info");

  const cg::BlobLayout bl = cg::blob_layout(L, C, info.n_groups, coded);
  const size_t cuts[] = {0, 1, 63, 64, 65, bl.off_pay, blob.size() - 17, blob.size() - 1};
  for (size_t n : cuts) {
    std::vector<uint8_t> b(blob.begin(), blob.begin() + n);
    const int rc = cg_chunk_info_parse(b.data(), n, &info);
    expect(n >= 64 ? rc == CG_OK : rc == CG_E_INVAL, "blob header of a truncated blob");
    expect(oracle_decode(tab, b.data(), n, &corrupt) != 0, "oracle rejects a truncated blob");
  }

  struct Field {
    size_t off;
    uint32_t value;
  };
  const Field fields[] = {{0, 0x324B4743u}, {4, 1}, {4, 4}, {8, 0}, {8, 5000}, {12, 0},
                          {16, 0}, {20, 0xFFFFFFFFu}, {20, 60}, {24, 0}, {24, 100000},
                          {28, 0}, {32, 999}, {36, 3}, {40, 0x40000000u}, {44, 14}};
  for (const Field& f : fields) {
    std::vector<uint8_t> b(blob);
    put32(b, f.off, f.value);
    expect(cg_chunk_info_parse(b.data(), b.size(), &info) != CG_OK,
           "blob header field at " + std::to_string(f.off) + " rejected");
    expect(oracle_decode(tab, b.data(), b.size(), &corrupt) != 0,
           "oracle rejects blob header field at " + std::to_string(f.off));
  }
  {
    // a quality the tables hold but a different chunk geometry: the oracle
    // checks the blob against the tables
    std::vector<uint8_t> b(blob);
    put32(b, 20, CH);  // token offset of chunk 1 with chunk 0's token count: consistent header
    expect(cg_chunk_info_parse(b.data(), b.size(), &info) == CG_OK, "header of a moved chunk");
    expect(oracle_decode(tab, b.data(), b.size(), &corrupt) == 0, "oracle decodes a moved chunk");
  }
  {
    std::vector<uint8_t> b(blob);
    b[48] ^= 1;
    expect(oracle_decode(tab, b.data(), b.size(), &corrupt) != 0, "oracle: other tables id");
  }
  {
    // the other format version: a valid header of another layout, refused by
    // the tables
    std::vector<uint8_t> b(blob);
    put32(b, 4, coded ? 2u : 3u);
    expect(cg_chunk_info_parse(b.data(), b.size(), &info) == CG_OK && info.blob_bytes != blob.size(),
           "header of the other format version");
    expect(oracle_decode(tab, b.data(), b.size(), &corrupt) != 0, "oracle: other format version");
  }

  // lengths and row offsets that point past the payload
  {
    std::vector<uint8_t> b(blob);
    const uint16_t big = 0xFFFF;
    memcpy(b.data() + bl.off_len + 2 * 3, &big, 2);
    expect(oracle_decode(tab, b.data(), b.size(), &corrupt) == 0 && corrupt,
           "oracle flags a stream longer than the payload");
  }
  {
    std::vector<uint8_t> b(blob);
    put32(b, bl.off_rows + 4, 0xFFFFFFF0u);
    expect(oracle_decode(tab, b.data(), b.size(), &corrupt) == 0 && corrupt,
           "oracle flags a row offset past the payload");
  }
  {
    std::vector<uint8_t> b(blob);
    memset(b.data() + bl.off_len, 0, 2 * (size_t)bl.rows * C);
    expect(oracle_decode(tab, b.data(), b.size(), &corrupt) == 0 && corrupt,
           "oracle flags streams of zero length");
  }

  // random damage past the header: decoded or flagged, never a fault
  Rng r{777};
  int flagged = 0;
  for (int i = 0; i < 3000; i++) {
    std::vector<uint8_t> b(blob);
    const int nflip = 1 + (int)r.below(4);
    for (int j = 0; j < nflip; j++) {
      const size_t at = 64 + r.below(b.size() - 64);
      b[at] ^= (uint8_t)(1u << r.below(8));
    }
    expect(cg_chunk_info_parse(b.data(), b.size(), &info) == CG_OK, "header untouched by the damage");
    corrupt = 0;
    expect(oracle_decode(tab, b.data(), b.size(), &corrupt) == 0, "oracle decodes a damaged body");
    flagged += corrupt;
  }
  expect(flagged > 0, "some damaged bodies are flagged corrupt");
}

}  // namespace

int main() {
  params_cases();
  plan_cases();
  std::vector<uint16_t> k, v;
  make_kv(k, v);
  // raw anchors (tables version 1, blobs version 2), then coded anchors
  // (tables version 2, blobs version 3)
  for (int coded = 0; coded < 2; coded++) {
    const cgo_params op = oracle_params(coded);
    std::vector<uint8_t> tab(cgo_tables_size(&op));
    size_t tlen = 0;
    expect(cgo_build_tables(&op, k.data(), v.data(), 1, tab.data(), tab.size(), &tlen, nullptr) == 0 &&
               tlen == tab.size(),
           "oracle builds the tables");
    std::vector<uint8_t> blob(cgo_encode_bound(tab.data(), tab.size(), 0));
    size_t blen = 0;
    expect(cgo_encode_chunk(tab.data(), tab.size(), k.data(), v.data(), 0, 1, 1, blob.data(),
                            blob.size(), &blen) == 0,
           "oracle encodes chunk 0");
    blob.resize(blen);
    table_cases(tab, blob.data(), blob.size(), coded);
    unbalanced_frequency_case(tab, blob, coded);
    blob_cases(tab, blob, coded);
  }
  if (g_failures) {
    fprintf(stderr, "fault corpus: %d of %d cases failed\n", g_failures, g_cases);
    return 1;
  }
  printf("fault corpus ok: %d cases\n", g_cases);
  return 0;
}
