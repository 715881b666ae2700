// Host side of the C ABI declared in include/cachegen.h: argument validation,
// device memory, kernel launches, table (de)serialization and the chunk
// pipeline.  Every step of the codec runs in the kernels of cg_*.hip.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "cg_build.h"

using namespace cg;

struct cg_tables {
  cg_params p{};
  int dev = 0;
  DevTables t;
  uint64_t id = 0;
  std::mutex mu;  // guards the decode status words
  uint8_t* dev_block = nullptr;  // one allocation: serialized tables, images, status words
  uint32_t* status = nullptr;    // device words: decode status
  uint32_t* host_status = nullptr;  // pinned mirror, allocated on first use
};

namespace {

int hip_fail(hipError_t e, const char* what) {
  return fail(CG_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define HIP_TRY(expr, what)               \
  do {                                    \
    hipError_t e_ = (expr);               \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

void init_dev_tables(DevTables& t, const cg_params& p) {
  t.L = p.layers;
  t.T = p.tokens;
  t.C = p.channels;
  t.CH = p.chunk_tokens;
  t.G = p.group_tokens;
  t.nblk = (p.channels + kLanes - 1) / kLanes;
  t.mask = p.quality_mask;
  t.lay = tab_layout(p.layers, p.channels, p.quality_mask, p.anchor_coding != 0);
}

size_t img_bytes(const DevTables& t) { return (size_t)2 * t.L * t.nblk * kImgRows * kLanes * 2; }

void write_header(uint8_t* h, const cg_params& p) {
  memset(h, 0, kTabHdr);
  uint32_t u[20] = {0};
  u[0] = kTabMagic;
  u[1] = p.anchor_coding ? kTabVersionCoded : kTabVersion;
  u[2] = (uint32_t)p.layers;
  u[3] = (uint32_t)p.channels;
  u[4] = (uint32_t)p.tokens;
  u[5] = (uint32_t)p.chunk_tokens;
  u[6] = (uint32_t)p.group_tokens;
  u[7] = (uint32_t)p.n_layer_groups;
  for (int i = 0; i < 3; i++) {
    u[8 + i] = i < p.n_layer_groups ? (uint32_t)p.layer_group_end[i] : 0u;
    const float ls = i < p.n_layer_groups ? p.layer_step[i] : 0.0f;
    const float qm = ((p.quality_mask >> i) & 1) ? p.quality_mult[i] : 0.0f;
    memcpy(&u[11 + i], &ls, 4);
    memcpy(&u[14 + i], &qm, 4);
  }
  u[17] = p.quality_mask;
  u[18] = kProbBits;
  u[19] = kNSym;
  memcpy(h, u, kTabHdr);
}

constexpr int kMaxDevices = 64;

// Stream-ordered memory pool, one per device, made on first use and kept, with
// the blocks it has cached, until the process ends: the device copies of each
// tables handle and the coded-anchor decode workspaces come from it.  The
// device's default pool hands freed blocks back to the driver at the next
// synchronisation, and the next hipMalloc on the device then waits for that
// (about 0.4 ms after a coded-anchor decode); a hipMalloc of the tables' 75 MB
// of the Mistral-7B shape took 0.05-0.16 ms of every build.  This pool keeps
// what it has held (the high-water mark of the blocks outstanding at once).
struct KeepPool {
  std::mutex mu;
  hipMemPool_t pool = nullptr;
};

KeepPool* keep_pool_of(int dev) {
  static KeepPool p[kMaxDevices];
  return dev >= 0 && dev < kMaxDevices ? &p[dev] : nullptr;
}

int keep_pool(int dev, hipMemPool_t* out) {
  KeepPool* p = keep_pool_of(dev);
  if (!p) return fail(CG_E_INVAL, "device index beyond the supported range");
  std::lock_guard<std::mutex> lock(p->mu);
  if (!p->pool) {
    hipMemPoolProps props;
    memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    HIP_TRY(hipMemPoolCreate(&pool, &props), "hipMemPoolCreate");
    uint64_t keep = UINT64_MAX;
    const hipError_t e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return hip_fail(e, "hipMemPoolSetAttribute");
    }
    p->pool = pool;
  }
  *out = p->pool;
  return CG_OK;
}

void free_tables(cg_tables* t) {
  if (!t) return;
  DeviceGuard g(t->dev);
  if (t->dev_block) {
    // no work on any stream may still use the block (as hipFree would wait)
    (void)hipDeviceSynchronize();
    (void)hipFreeAsync(t->dev_block, nullptr);
  }
  if (t->host_status) (void)hipHostFree(t->host_status);
  delete t;
}

// Allocates the device copies of a table set whose params are already checked.
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// The tables' device memory in one allocation: serialized tables, the LDS
// images of each built quality, 64 status words.
int alloc_tables(cg_tables* h, hipStream_t st) {
  DevTables& t = h->t;
  size_t off = align256(t.lay.total);
  size_t img_off[3] = {0, 0, 0};
  for (int q = 0; q < 3; q++)
    if ((t.mask >> q) & 1u) {
      img_off[q] = off;
      off += align256(img_bytes(t));
    }
  const size_t status_off = off;
  off += 256;
  hipMemPool_t pool = nullptr;
  if (int rc = keep_pool(h->dev, &pool)) return rc;
  HIP_TRY(hipMallocFromPoolAsync((void**)&h->dev_block, off, pool, st), "tables allocation");
  t.ser = h->dev_block;
  for (int q = 0; q < 3; q++)
    if ((t.mask >> q) & 1u) t.img[q] = reinterpret_cast<uint16_t*>(h->dev_block + img_off[q]);
  h->status = reinterpret_cast<uint32_t*>(h->dev_block + status_off);
  return CG_OK;
}

int ensure_host_status(cg_tables* h) {
  if (!h->host_status)
    HIP_TRY(hipHostMalloc(&h->host_status, 64, hipHostMallocDefault), "hipHostMalloc(status)");
  return CG_OK;
}

// Device workspace of cg_build_tables and of the tables id (statistics, symbol
// counts, digests) and a pinned word block for reading back status and id:
// one per device, grown when a build needs more and kept until the process
// ends.  A build holds the mutex until it has synchronised its stream, so
// builds on one device take turns.
struct BuildWs {
  std::mutex mu;
  uint8_t* dev = nullptr;
  size_t bytes = 0;
  uint32_t* host = nullptr;
};

BuildWs* build_ws(int dev) {
  static BuildWs ws[kMaxDevices];
  return dev >= 0 && dev < kMaxDevices ? &ws[dev] : nullptr;
}

// with ws->mu held
int reserve_ws(BuildWs* ws, size_t bytes) {
  if (!ws->host) HIP_TRY(hipHostMalloc(&ws->host, 64, hipHostMallocDefault), "hipHostMalloc(build)");
  if (ws->bytes >= bytes) return CG_OK;
  if (ws->dev) (void)hipFree(ws->dev);
  ws->dev = nullptr;
  ws->bytes = 0;
  if (hipMalloc(&ws->dev, bytes) != hipSuccess)
    return fail(CG_E_NOMEM, "device allocation for the table build workspace");
  ws->bytes = bytes;
  return CG_OK;
}

size_t id_digest_bytes(const DevTables& t) {
  return 8 * (id_leaves(t.lay.total) + id_mids(t.lay.total));
}

// Tables id of the device copy, computed on the GPU; syncs the stream.
int compute_id(cg_tables* h, hipStream_t st) {
  BuildWs* ws = build_ws(h->dev);
  if (!ws) return fail(CG_E_INVAL, "device index beyond the supported range");
  std::lock_guard<std::mutex> lock(ws->mu);
  int rc = reserve_ws(ws, id_digest_bytes(h->t) + 8);
  if (rc) return rc;
  uint64_t* dig = reinterpret_cast<uint64_t*>(ws->dev);
  const size_t nd = id_digest_bytes(h->t) / 8;
  hipError_t e = launch_tables_id(h->t, dig, dig + nd, st);
  if (e == hipSuccess) e = hipMemcpyAsync(ws->host, dig + nd, 8, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "tables id");
  memcpy(&h->id, ws->host, 8);
  return CG_OK;
}

struct ChunkGeo {
  int t0, tc, ng;
};

ChunkGeo chunk_geo(const DevTables& t, int chunk) {
  ChunkGeo g;
  g.t0 = chunk * t.CH;
  g.tc = std::min(t.CH, t.T - g.t0);
  g.ng = (g.tc + t.G - 1) / t.G;
  return g;
}

int n_chunks_of(const DevTables& t) { return (t.T + t.CH - 1) / t.CH; }

bool coded_anchors(const DevTables& t) { return t.lay.off_afreq != 0; }

// the layout of a blob of `ng` groups coded with these tables
BlobLayout blob_layout_of(const DevTables& t, int ng) {
  return blob_layout(t.L, t.C, ng, coded_anchors(t));
}

int check_info_against(const cg_tables* h, const cg_chunk_info& in) {
  const DevTables& t = h->t;
  if (in.layers != t.L || in.channels != t.C || in.total_tokens != t.T || in.group_tokens != t.G)
    return fail(CG_E_MISMATCH, "blob shape differs from the tables");
  if (in.tables_id != h->id) return fail(CG_E_MISMATCH, "blob was coded with other tables");
  if ((in.version == kBlobVersionCoded) != coded_anchors(t))
    return fail(CG_E_MISMATCH, "blob format differs from the tables' anchor coding");
  if (!((t.mask >> in.quality) & 1u)) return fail(CG_E_MISMATCH, "quality not in the tables");
  if (in.token_offset % t.CH) return fail(CG_E_INVAL, "token_offset is not a chunk start");
  const ChunkGeo g = chunk_geo(t, in.token_offset / t.CH);
  if (g.tc != in.chunk_tokens) return fail(CG_E_INVAL, "chunk_tokens differs from the geometry");
  return CG_OK;
}

// Where a paged decode writes (arguments already checked).
struct PagedOut {
  const int32_t* table;
  uint32_t n_blocks, num_pages, shift;
};

// The decode launches of n blobs whose headers are already checked, into
// [L][T][C] tensors or, with pg, into paged pools; anc[i] = blob i's anchors
// (i8 [2][L][ng][C]).
int enqueue_decode_chunks(const cg_tables* h, int n, const void* const* blobs,
                          const cg_chunk_info* infos, const int8_t* const* anc, void* k_out,
                          void* v_out, uint32_t* status, hipStream_t st, const PagedOut* pg) {
  const DevTables& t = h->t;
  // chunks grouped by quality, up to 4 per workgroup (one wave per chunk and kv)
  std::vector<int> byq[3];
  for (int i = 0; i < n; i++) byq[infos[i].quality].push_back(i);
  std::vector<std::vector<int>> groups;
  for (int q = 0; q < 3; q++)
    for (size_t j = 0; j < byq[q].size(); j += 4) {
      std::vector<int> g(byq[q].begin() + j, byq[q].begin() + std::min(byq[q].size(), j + 4));
      groups.push_back(g);
    }
  size_t gi = 0;
  while (gi < groups.size()) {
    DecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.L = t.L;
    a.T = t.T;
    a.C = t.C;
    a.G = t.G;
    a.nblk = t.nblk;
    for (int q = 0; q < 3; q++) {
      a.img[q] = t.img[q];
      a.step[q] = ((t.mask >> q) & 1u) ? reinterpret_cast<const float*>(t.ser + t.lay.off_step[q])
                                       : nullptr;
    }
    a.scale_a = reinterpret_cast<const float*>(t.ser + t.lay.off_scale_a);
    a.k_out = static_cast<uint16_t*>(k_out);
    a.v_out = static_cast<uint16_t*>(v_out);
    a.status = status;
    if (pg) {
      a.paged = 1;
      a.block_table = pg->table;
      a.n_blocks = pg->n_blocks;
      a.num_pages = pg->num_pages;
      a.page_shift = pg->shift;
    }
    int nc = 0, ngrp = 0, waves = 1;
    while (gi < groups.size() && ngrp < kDecMaxChunks &&
           nc + (int)groups[gi].size() <= kDecMaxChunks) {
      DecGroup dg;
      for (int w = 0; w < 4; w++) dg.chunk[w] = -1;
      for (size_t w = 0; w < groups[gi].size(); w++) {
        const int i = groups[gi][w];
        const cg_chunk_info& in = infos[i];
        const BlobLayout bl = blob_layout_of(t, in.n_groups);
        DecChunk& dc = a.chunks[nc];
        dc.blob = static_cast<const uint8_t*>(blobs[i]);
        dc.blob_bytes = (uint32_t)in.blob_bytes;
        dc.t0 = in.token_offset;
        dc.tc = in.chunk_tokens;
        dc.ng = in.n_groups;
        dc.q = in.quality;
        dc.anc = anc[i];
        dc.anc_bytes = (uint32_t)((size_t)2 * t.L * in.n_groups * t.C);
        dc.off_len = (uint32_t)bl.off_len;
        dc.off_pay = (uint32_t)bl.off_pay;
        dc.W = in.payload_words;
        dg.chunk[w] = (int8_t)nc++;
      }
      waves = std::max(waves, (int)groups[gi].size());
      a.groups[ngrp++] = dg;
      gi++;
    }
    a.n_groups = ngrp;
    a.waves = waves;
    // a warming wave where it pays and costs no decoding wave: two chunks per
    // workgroup (4 decoding waves, 26.9 KB of LDS, six workgroups per CU: 30 of
    // a CU's 32 wave slots with it); with three or four chunks it would take
    // slots the decoding waves fill, and one-chunk launches (the register-buffer
    // kernel) decoded no faster with it
    a.warm_wave = waves == 2 ? 1 : 0;
    HIP_TRY(launch_decode(a, st), "decode launch");
  }
  return CG_OK;
}

// Enqueues the decode of n checked blobs.  Raw anchors are read from the
// blobs; coded anchors are first decoded into a stream-ordered allocation of
// 2 L ng C bytes per blob from the device's anchor pool (allocated on st,
// freed on st after the decode).
int enqueue_decode(const cg_tables* h, int n, const void* const* blobs, const cg_chunk_info* infos,
                   void* k_out, void* v_out, uint32_t* status, hipStream_t st,
                   const PagedOut* pg = nullptr) {
  const DevTables& t = h->t;
  std::vector<const int8_t*> anc(n);
  if (!coded_anchors(t)) {
    for (int i = 0; i < n; i++)
      anc[i] = reinterpret_cast<const int8_t*>(blobs[i]) + blob_layout_of(t, infos[i].n_groups).off_anchor;
    return enqueue_decode_chunks(h, n, blobs, infos, anc.data(), k_out, v_out, status, st, pg);
  }
  std::vector<size_t> off(n);
  size_t bytes = 0;
  for (int i = 0; i < n; i++) {
    off[i] = bytes;
    bytes += align256((size_t)2 * t.L * infos[i].n_groups * t.C);
  }
  hipMemPool_t pool = nullptr;
  int rc = keep_pool(h->dev, &pool);
  if (rc) return rc;
  int8_t* ws = nullptr;
  HIP_TRY(hipMallocFromPoolAsync((void**)&ws, bytes, pool, st), "hipMallocFromPoolAsync(anchors)");
  for (int i0 = 0; i0 < n && rc == CG_OK; i0 += kDecMaxChunks) {
    AnchorDecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.L = t.L;
    a.C = t.C;
    a.nblk = t.nblk;
    a.nchunks = std::min(kDecMaxChunks, n - i0);
    a.afreq = reinterpret_cast<const uint16_t*>(t.ser + t.lay.off_afreq);
    a.status = status;
    for (int j = 0; j < a.nchunks; j++) {
      const cg_chunk_info& in = infos[i0 + j];
      const BlobLayout bl = blob_layout_of(t, in.n_groups);
      AncChunk& c = a.chunks[j];
      c.blob = static_cast<const uint8_t*>(blobs[i0 + j]);
      c.blob_bytes = (uint32_t)in.blob_bytes;
      c.ng = in.n_groups;
      c.off_len = (uint32_t)bl.off_len;
      c.off_pay = (uint32_t)bl.off_pay;
      c.W = in.payload_words;
      c.out = ws + off[i0 + j];
    }
    const hipError_t e = launch_anchor_decode(a, st);
    if (e != hipSuccess) rc = hip_fail(e, "anchor decode launch");
  }
  for (int i = 0; i < n; i++) anc[i] = ws + off[i];
  if (rc == CG_OK)
    rc = enqueue_decode_chunks(h, n, blobs, infos, anc.data(), k_out, v_out, status, st, pg);
  const hipError_t e = hipFreeAsync(ws, st);
  if (rc == CG_OK && e != hipSuccess) rc = hip_fail(e, "hipFreeAsync(anchors)");
  return rc;
}

// Arguments of an encode batch, checked before any launch.
int check_encode_args(const cg_tables* h, const void* k_dev, const void* v_dev, int32_t n,
                      const int32_t* chunks, const int32_t* qualities, void* const* outs_dev,
                      const size_t* caps, size_t* out_lens) {
  if (!h || !k_dev || !v_dev || n < 0 || (n > 0 && (!chunks || !qualities || !outs_dev ||
                                                     !caps || !out_lens)))
    return fail(CG_E_INVAL, "NULL argument");
  const DevTables& t = h->t;
  for (int i = 0; i < n; i++) {
    if (!outs_dev[i]) return fail(CG_E_INVAL, "NULL output");
    if (chunks[i] < 0 || chunks[i] >= n_chunks_of(t)) return fail(CG_E_INVAL, "chunk out of range");
    if (qualities[i] < 0 || qualities[i] > 2 || !((t.mask >> qualities[i]) & 1u))
      return fail(CG_E_MISMATCH, "quality not in the tables");
    const ChunkGeo g = chunk_geo(t, chunks[i]);
    if (caps[i] < blob_layout_of(t, g.ng).off_pay + 16)
      return fail(CG_E_CAPACITY, "output smaller than the blob's fixed part");
  }
  return CG_OK;
}

// Scratch words of one stream: its worst-case words in whole 16-byte units
// (every chunk of the tables fits the longest chunk's bound).
size_t stream_scratch_words(const DevTables& t) {
  return (std::max<size_t>(stream_words_bound(t.CH - (t.CH + t.G - 1) / t.G), 1) + 3) & ~(size_t)3;
}

// the same for an anchor stream (one symbol per group), 0 without coded anchors
size_t anchor_scratch_words(const DevTables& t) {
  return coded_anchors(t) ? (std::max<size_t>(stream_words_bound((t.CH + t.G - 1) / t.G), 1) + 3) & ~(size_t)3
                          : 0;
}

// The fields of one blob of an encode launch, but for its scratch buffers.
void init_enc_blob(EncBlob& B, const DevTables& t, int chunk, int q, void* out, size_t cap) {
  const ChunkGeo g = chunk_geo(t, chunk);
  B.blob = static_cast<uint8_t*>(out);
  B.cap = cap;
  B.t0 = g.t0;
  B.tc = g.tc;
  B.ng = g.ng;
  B.q = q;
  B.lay = blob_layout_of(t, g.ng);
  B.img = t.img[q];
  B.inv_step = reinterpret_cast<const float*>(t.ser + t.lay.off_inv_step[q]);
}

// The launch-wide fields of an encode launch.
void init_enc_args(EncodeArgs& a, const cg_tables* h, const void* k_dev, const void* v_dev,
                   size_t swb) {
  const DevTables& t = h->t;
  memset(&a, 0, sizeof(a));
  a.k = static_cast<const uint16_t*>(k_dev);
  a.v = static_cast<const uint16_t*>(v_dev);
  a.L = t.L;
  a.T = t.T;
  a.C = t.C;
  a.G = t.G;
  a.nblk = t.nblk;
  a.swb = swb;
  a.scale_a = reinterpret_cast<const float*>(t.ser + t.lay.off_scale_a);
  a.inv_a = reinterpret_cast<const float*>(t.ser + t.lay.off_inv_a);
  a.tables_id = h->id;
  a.row0 = 0;
  a.nrows = 2 * t.L;
  a.rows_total = coded_anchors(t) ? 4 * t.L : 2 * t.L;
  a.afreq = coded_anchors(t) ? reinterpret_cast<const uint16_t*>(t.ser + t.lay.off_afreq) : nullptr;
  a.waves = 1;
  int cus = 0, lds = 0;
  a.ncu = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->dev) == hipSuccess && cus > 0
              ? cus : 1;
  a.lds_cu = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, h->dev) ==
                     hipSuccess && lds > 0
                 ? lds : 65536;
}

// out_lens[i] and the call's result from blob i's status words {payload words,
// too large, non-finite}; rc keeps the first failure.
void finish_blob(const DevTables& t, int chunk, const uint32_t* sw, size_t* out_len, int* rc) {
  *out_len = 0;
  if (sw[2]) {
    if (*rc == CG_OK) *rc = fail(CG_E_INVAL, "K/V hold a non-finite value");
  } else if (sw[1]) {
    if (*rc == CG_OK) *rc = fail(CG_E_CAPACITY, "blob larger than the output buffer");
  } else {
    *out_len = blob_bytes(blob_layout_of(t, chunk_geo(t, chunk).ng), sw[0]);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// The static encode scratch of cg_encode_batch_noalloc: device memory that
// exists, one copy per GPU, from the code object's load until the process
// ends, so that the call allocates nothing.  In host code the array's name is
// a host-side stand-in, not a device address: host code reaches the array only
// through the address hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticScratchBytes = (size_t)256 << 20;
static __device__ __align__(256) uint32_t scratch[kStaticScratchBytes / 4];

namespace {

struct StaticScratch {
  std::mutex mu;            // held by a call until its stream has finished
  uint32_t* ptr = nullptr;  // device address of this device's array
};

StaticScratch* static_scratch(int dev) {
  static StaticScratch s[kMaxDevices];
  return dev >= 0 && dev < kMaxDevices ? &s[dev] : nullptr;
}

// The device address of the array on the current device (with s->mu held):
// looked up once per device, on the first call there.
int static_scratch_ptr(StaticScratch* s, uint32_t** out) {
  if (!s->ptr) {
    uint32_t* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    s->ptr = ptr;
  }
  *out = s->ptr;
  return CG_OK;
}

size_t align64w(size_t words) { return (words + 63) & ~(size_t)63; }

}  // namespace

extern "C" {

int cg_build_tables(const cg_params* params, const void* k_dev, const void* v_dev, void* stream,
                    cg_tables** out) {
  return cg_build_tables_grouped(params, CG_GROUP_LAYER_CHANNEL, k_dev, v_dev, stream, out);
}

int cg_build_tables_grouped(const cg_params* params_in, int32_t grouping, const void* k_dev,
                            const void* v_dev, void* stream, cg_tables** out) {
  cg_params resolved;
  int rc = resolve_params(params_in, &resolved);
  if (rc) return rc;
  const cg_params* params = &resolved;
  rc = check_params(params);
  if (rc) return rc;
  if (grouping < CG_GROUP_LAYER_CHANNEL || grouping > CG_GROUP_GLOBAL)
    return fail(CG_E_INVAL, "unknown table grouping");
  if (!k_dev || !v_dev || !out) return fail(CG_E_INVAL, "NULL argument");
  *out = nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  cg_tables* h = new (std::nothrow) cg_tables();
  if (!h) return fail(CG_E_NOMEM, "host allocation");
  h->p = *params;
  if (hipGetDevice(&h->dev) != hipSuccess) {
    delete h;
    return fail(CG_E_HIP, "no HIP device");
  }
  init_dev_tables(h->t, *params);
  DevTables& t = h->t;
  if ((rc = alloc_tables(h, st))) {
    free_tables(h);
    return rc;
  }
  const size_t n = t.lay.n;
  const size_t counts_words = (size_t)n * t.lay.nq * kNSym;
  const size_t acounts_words = t.lay.off_afreq ? (size_t)2 * t.L * kASym : 0;
  // workspace: [s1 | sa | sc] u64, amax u32, 8 flag words (2 and 3 hold the
  // tables id), counts, anchor counts; then the id digests, then pooled counts
  const size_t tmp_bytes = 3 * 8 * n + 4 * n + 32 + 4 * (counts_words + acounts_words);
  const size_t dig_off = align256(tmp_bytes);
  const size_t pool_off = align256(dig_off + id_digest_bytes(t));
  const size_t pool_bytes = grouping ? 4 * pooled_words(t, grouping) : 0;
  BuildWs* ws = build_ws(h->dev);
  if (!ws) {
    free_tables(h);
    return fail(CG_E_INVAL, "device index beyond the supported range");
  }
  std::lock_guard<std::mutex> lock(ws->mu);
  if ((rc = reserve_ws(ws, pool_off + pool_bytes))) {
    free_tables(h);
    return rc;
  }
  uint8_t* tmp = ws->dev;
  StatsBuf sb;
  sb.s1 = reinterpret_cast<uint64_t*>(tmp);
  sb.sa = sb.s1 + n;
  sb.sc = sb.sa + n;
  sb.amax = reinterpret_cast<uint32_t*>(sb.sc + n);
  sb.flags = sb.amax + n;
  uint64_t* id_dev = reinterpret_cast<uint64_t*>(sb.flags + 2);
  uint32_t* counts = sb.flags + 8;
  uint32_t* acounts = counts + counts_words;
  uint64_t* dig = reinterpret_cast<uint64_t*>(tmp + dig_off);
  uint32_t* pooled = reinterpret_cast<uint32_t*>(tmp + pool_off);
  uint8_t hdr[kTabHdr];
  write_header(hdr, *params);
  const uint16_t* k = static_cast<const uint16_t*>(k_dev);
  const uint16_t* v = static_cast<const uint16_t*>(v_dev);
  hipError_t e = hipMemsetAsync(tmp, 0, tmp_bytes, st);
  if (e == hipSuccess) e = hipMemcpyAsync(t.ser, hdr, kTabHdr, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = launch_stats(k, 0, t.L, t.T, t.C, sb, st);
  if (e == hipSuccess) e = launch_stats(v, 1, t.L, t.T, t.C, sb, st);
  if (e == hipSuccess) e = launch_finalize(*params, sb, t, st);
  if (e == hipSuccess) e = launch_histogram(k, 0, t, counts, acounts, st);
  if (e == hipSuccess) e = launch_histogram(v, 1, t, counts, acounts, st);
  if (e == hipSuccess && grouping) e = launch_pool(t, counts, grouping, pooled, sb.flags + 4, st);
  if (e == hipSuccess) e = launch_normalize(t, counts, st);
  if (e == hipSuccess) e = launch_normalize_anchors(t, acounts, st);
  if (e == hipSuccess) e = launch_images(t, st);
  // the id of whatever was built; discarded below when the build failed
  if (e == hipSuccess) e = launch_tables_id(t, dig, id_dev, st);
  if (e == hipSuccess) e = hipMemcpyAsync(ws->host, sb.flags, 32, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    free_tables(h);
    return hip_fail(e, "build tables");
  }
  if (ws->host[0]) {
    free_tables(h);
    return fail(CG_E_INVAL, "K/V hold a non-finite value");
  }
  if (ws->host[1]) {
    free_tables(h);
    return fail(CG_E_INVAL, "a delta step is not a normal binary32 value");
  }
  if (ws->host[4]) {
    free_tables(h);
    return fail(CG_E_INVAL, "a pooled symbol count does not fit 32 bits");
  }
  memcpy(&h->id, ws->host + 2, 8);
  *out = h;
  return CG_OK;
}

void cg_tables_free(cg_tables* tables) { free_tables(tables); }

int cg_tables_serialize(const cg_tables* h, void* buf, size_t cap, size_t* len) {
  if (!h || !len) return fail(CG_E_INVAL, "NULL argument");
  *len = h->t.lay.total;
  if (!buf) return CG_OK;
  if (cap < h->t.lay.total) return fail(CG_E_CAPACITY, "buffer smaller than the tables");
  DeviceGuard g(h->dev);
  HIP_TRY(hipMemcpy(buf, h->t.ser, h->t.lay.total, hipMemcpyDeviceToHost), "copy tables");
  return CG_OK;
}

int cg_tables_deserialize(const void* buf, size_t len, cg_tables** out) {
  if (!buf || !out) return fail(CG_E_INVAL, "NULL argument");
  *out = nullptr;
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  cg_params p;
  int rc = check_tables_image(b, len, &p);
  if (rc) return rc;
  cg_tables* h = new (std::nothrow) cg_tables();
  if (!h) return fail(CG_E_NOMEM, "host allocation");
  h->p = p;
  if (hipGetDevice(&h->dev) != hipSuccess) {
    delete h;
    return fail(CG_E_HIP, "no HIP device");
  }
  init_dev_tables(h->t, p);
  if ((rc = alloc_tables(h, nullptr))) {
    free_tables(h);
    return rc;
  }
  hipError_t e = hipMemcpy(h->t.ser, b, len, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = launch_images(h->t, nullptr);
  if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) {
    free_tables(h);
    return hip_fail(e, "upload tables");
  }
  if ((rc = compute_id(h, nullptr))) {
    free_tables(h);
    return rc;
  }
  *out = h;
  return CG_OK;
}

uint64_t cg_tables_id(const cg_tables* h) { return h ? h->id : 0; }

int cg_tables_params(const cg_tables* h, cg_params* out) {
  if (!h || !out) return fail(CG_E_INVAL, "NULL argument");
  *out = h->p;
  return CG_OK;
}

int cg_num_chunks(const cg_tables* h, int32_t* n) {
  if (!h || !n) return fail(CG_E_INVAL, "NULL argument");
  *n = n_chunks_of(h->t);
  return CG_OK;
}

int cg_encode_bound(const cg_tables* h, int32_t chunk, size_t* max_bytes) {
  if (!h || !max_bytes) return fail(CG_E_INVAL, "NULL argument");
  if (chunk < 0 || chunk >= n_chunks_of(h->t)) return fail(CG_E_INVAL, "chunk out of range");
  const ChunkGeo g = chunk_geo(h->t, chunk);
  const BlobLayout bl = blob_layout_of(h->t, g.ng);
  size_t words = h->t.lay.n * stream_words_bound(g.tc - g.ng);
  if (coded_anchors(h->t)) words += h->t.lay.n * stream_words_bound(g.ng);
  *max_bytes = blob_bytes(bl, words);
  return CG_OK;
}

// Scratch memory the encoder may hold: the blobs of one launch share it.
constexpr size_t kEncScratchBudget = (size_t)3 << 30;

// Device workspace of cg_encode_batch, one per device, grown when a batch needs
// more and kept until the process ends: per blob slot of a launch the streams'
// scratch ([2][L][nblk] blocks of [swb][64] words), their lengths ([2][L][C])
// and row and block totals ([2L], then [2L][nblk]); per blob of a batch four
// status words (W, too large, non-finite, pad) and their pinned mirror.  A
// batch holds the mutex until it has synchronised its stream, so batches on
// one device take turns.  (Allocated per tables handle, the 1 GB of scratch of
// an 18-blob Mistral-7B-shape batch cost 0.2 ms of hipMalloc, with the GPU
// idle, in the first batch on every new tables handle.)
struct EncWs {
  std::mutex mu;
  uint32_t* scratch = nullptr;
  size_t scratch_bytes = 0;
  uint32_t* lens = nullptr;
  size_t lens_bytes = 0;
  uint32_t* row_words = nullptr;
  size_t row_bytes = 0;
  uint32_t* status = nullptr;
  uint32_t* host = nullptr;
  size_t status_bytes = 0;
};

EncWs* enc_ws(int dev) {
  static EncWs ws[kMaxDevices];
  return dev >= 0 && dev < kMaxDevices ? &ws[dev] : nullptr;
}

// with ws->mu held: *buf holds at least `bytes` device bytes
int reserve_dev(uint32_t** buf, size_t* have, size_t bytes) {
  if (*have >= bytes) return CG_OK;
  if (*buf) (void)hipFree(*buf);
  *buf = nullptr;
  *have = 0;
  if (hipMalloc(buf, bytes) != hipSuccess) return fail(CG_E_NOMEM, "encode workspace");
  *have = bytes;
  return CG_OK;
}

// Waves the device can hold at once: compute units x threads per compute unit
// / 64 (the encoder's VGPR and LDS use leave this bound the binding one).
size_t resident_waves(int dev) {
  int cus = 0, threads = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&threads, hipDeviceAttributeMaxThreadsPerMultiProcessor, dev) != hipSuccess ||
      cus <= 0 || threads <= 0)
    return (size_t)1 << 30;  // unknown: no cap from this bound
  return (size_t)cus * (size_t)threads / kLanes;
}

int cg_encode_batch(const cg_tables* ch, const void* k_dev, const void* v_dev, int32_t n,
                    const int32_t* chunks, const int32_t* qualities, void* const* outs_dev,
                    const size_t* caps, size_t* out_lens, void* stream) {
  int rc = check_encode_args(ch, k_dev, v_dev, n, chunks, qualities, outs_dev, caps, out_lens);
  if (rc) return rc;
  if (n == 0) return CG_OK;
  cg_tables* h = const_cast<cg_tables*>(ch);
  const DevTables& t = h->t;
  DeviceGuard dg(h->dev);
  if (!dg.ok) return fail(CG_E_HIP, "cannot select the tables' device");
  EncWs* ws = enc_ws(h->dev);
  if (!ws) return fail(CG_E_INVAL, "device index beyond the supported range");
  std::lock_guard<std::mutex> lk(ws->mu);
  const size_t swb = stream_scratch_words(t), aswb = anchor_scratch_words(t);
  // whole 64-stream blocks of 2L rows: the delta rows, then (coded anchors) the
  // anchor rows in the same buffers
  const size_t slot_words = (size_t)2 * t.L * t.nblk * kLanes * std::max(swb, aswb);
  // Blobs per launch: at most what the scratch budget holds.  When one more
  // launch is enough to make every launch fit the device at once (a blob is
  // 2 L nblk waves), take that, so that no second round of a few waves per
  // SIMD trails a launch and the waves' progress can be levelled.
  const size_t cap = resident_waves(h->dev);
  const size_t wpb = (size_t)2 * t.L * t.nblk;
  const size_t budget = std::max<size_t>(
      1, std::min<size_t>({(size_t)kEncMaxBlobs, (size_t)n, kEncScratchBudget / (4 * slot_words)}));
  const size_t fit = std::max<size_t>(1, std::min(budget, cap / wpb));
  const bool one_round = (n + fit - 1) / fit <= (n + budget - 1) / budget + 1;
  int slots = (int)(one_round ? fit : budget);
  // The encoder stages its output in rings of 8 words per lane, 2 KB a wave of
  // LDS beside the workgroup's 8 KB table, where all the launch's workgroups
  // fit their compute units with them (else it takes 4-word rings and checks
  // for complete units every symbol).  When they would not with `slots` blobs
  // but would with a smaller multiple of 4 (whole groups of one quality), take
  // that.
  {
    int cus = 0, lds = 0;
    if (slots > 4 && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->dev) == hipSuccess &&
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, h->dev) == hipSuccess &&
        cus > 0 && lds > 0) {
      auto fits8 = [&](size_t b) {
        const size_t wgs = (b + 3) / 4 * 2 * (size_t)t.L * t.nblk;
        const size_t per_wg = 2u * kImgRows * kLanes + std::min<size_t>(4, b) * 8u * 256u;
        return (wgs + (size_t)cus - 1) / (size_t)cus * per_wg <= (size_t)lds;
      };
      if (!fits8((size_t)slots)) {
        size_t b = (size_t)slots / 4 * 4;
        while (b >= 4 && !fits8(b)) b -= 4;
        if (b >= 4) slots = (int)b;
      }
    }
  }
  const size_t row_words_per_slot = (size_t)2 * t.L * (1 + t.nblk);
  if ((rc = reserve_dev(&ws->scratch, &ws->scratch_bytes, 4 * slot_words * slots)) ||
      (rc = reserve_dev(&ws->lens, &ws->lens_bytes, 4 * t.lay.n * slots)) ||
      (rc = reserve_dev(&ws->row_words, &ws->row_bytes, 4 * row_words_per_slot * slots)))
    return rc;
  if (ws->status_bytes < 16 * (size_t)n) {
    if (ws->status) (void)hipFree(ws->status);
    if (ws->host) (void)hipHostFree(ws->host);
    ws->status = ws->host = nullptr;
    ws->status_bytes = 0;
    if (hipMalloc(&ws->status, 16 * (size_t)n) != hipSuccess ||
        hipHostMalloc(&ws->host, 16 * (size_t)n, hipHostMallocDefault) != hipSuccess)
      return fail(CG_E_NOMEM, "encode status");
    ws->status_bytes = 16 * (size_t)n;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(hipMemsetAsync(ws->status, 0, 16 * (size_t)n, st), "clear status");
  // blobs in quality order, so that the blobs of one launch fall into few groups
  // of one quality (a group's workgroups stage each table once for all of them)
  std::vector<int> order(n);
  for (int i = 0; i < n; i++) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return qualities[x] < qualities[y]; });
  // launches of equal size (a small last launch would leave most of the GPU idle)
  const int launches = (n + slots - 1) / slots;
  const int per_launch = (n + launches - 1) / launches;
  for (int i0 = 0; i0 < n; i0 += per_launch) {
    EncodeArgs a;
    init_enc_args(a, h, k_dev, v_dev, swb);
    a.nblobs = std::min(per_launch, n - i0);
    a.prio = (size_t)a.nblobs * wpb <= cap ? 1 : 0;
    for (int j = 0; j < a.nblobs; j++) {
      const int i = order[i0 + j];
      EncBlob& B = a.b[j];
      init_enc_blob(B, t, chunks[i], qualities[i], outs_dev[i], caps[i]);
      B.scratch = ws->scratch + (size_t)j * slot_words;
      B.lens = ws->lens + (size_t)j * t.lay.n;
      B.row_words = ws->row_words + (size_t)j * row_words_per_slot;
      B.block_words = B.row_words + 2 * t.L;
      B.status = ws->status + 4 * (size_t)i;
      // open a new group at a quality change or when the current one is full
      if (j == 0 || a.b[j - 1].q != B.q || a.groups[a.n_groups - 1].blob[3] >= 0) {
        EncGroup& eg = a.groups[a.n_groups++];
        for (int w = 0; w < 4; w++) eg.blob[w] = -1;
      }
      EncGroup& eg = a.groups[a.n_groups - 1];
      int w = 0;
      while (eg.blob[w] >= 0) w++;
      eg.blob[w] = (int8_t)j;
      a.waves = std::max(a.waves, w + 1);
    }
    HIP_TRY(launch_encode(a, st), "encode launch");
    if (coded_anchors(t)) {
      // the anchor rows of the same blobs, through the same scratch
      a.row0 = 2 * t.L;
      a.swb = aswb;
      HIP_TRY(launch_encode(a, st), "anchor encode launch");
    }
  }
  HIP_TRY(hipMemcpyAsync(ws->host, ws->status, 16 * (size_t)n, hipMemcpyDeviceToHost, st),
          "encode status");
  HIP_TRY(hipStreamSynchronize(st), "encode");
  rc = CG_OK;
  for (int i = 0; i < n; i++) finish_blob(t, chunks[i], ws->host + 4 * (size_t)i, &out_lens[i], &rc);
  return rc;
}

int cg_encode_batch_noalloc(const cg_tables* ch, const void* k_dev, const void* v_dev, int32_t n,
                            const int32_t* chunks, const int32_t* qualities,
                            void* const* outs_dev, const size_t* caps, size_t* out_lens,
                            void* stream) {
  int rc = check_encode_args(ch, k_dev, v_dev, n, chunks, qualities, outs_dev, caps, out_lens);
  if (rc) return rc;
  if (n == 0) return CG_OK;
  const DevTables& t = ch->t;
  // The array holds 64 status words, then for a range of (kv, layer) rows their
  // stream lengths, row and block totals and stream words; the range is as many
  // rows as fit, a blob is coded range after range.
  const size_t swb = stream_scratch_words(t), aswb = anchor_scratch_words(t);
  const size_t per_row = (size_t)t.C + 1 + t.nblk + (size_t)t.nblk * kLanes * std::max(swb, aswb);
  const size_t fixed = 64 + 3 * 63;  // status words and the ranges' alignment
  const size_t rows_fit = (kStaticScratchBytes / 4 - fixed) / per_row;
  if (rows_fit < 1)
    return fail(CG_E_CAPACITY, "one (kv, layer) row of a chunk needs " + std::to_string(4 * per_row) +
                                   " bytes of encode scratch; the static scratch holds " +
                                   std::to_string(kStaticScratchBytes));
  const int rows_max = (int)std::min<size_t>(rows_fit, (size_t)2 * t.L);
  DeviceGuard dg(ch->dev);
  if (!dg.ok) return fail(CG_E_HIP, "cannot select the tables' device");
  StaticScratch* ss = static_scratch(ch->dev);
  if (!ss) return fail(CG_E_INVAL, "device index beyond the supported range");
  std::lock_guard<std::mutex> lk(ss->mu);
  uint32_t* base = nullptr;
  if ((rc = static_scratch_ptr(ss, &base))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t cap = resident_waves(ch->dev);
  uint32_t* status = base;  // words 0..3 of blob i while it is coded
  rc = CG_OK;
  for (int i = 0; i < n; i++) {
    HIP_TRY(launch_zero_words(status, 4, st), "clear status");
    // delta rows 0 .. 2L-1, then (coded anchors) anchor rows 2L .. 4L-1; no
    // range straddles 2L
    const int rows_total = coded_anchors(t) ? 4 * t.L : 2 * t.L;
    for (int r0 = 0; r0 < rows_total;) {
      const int part_end = r0 < 2 * t.L ? 2 * t.L : rows_total;
      EncodeArgs a;
      init_enc_args(a, ch, k_dev, v_dev, r0 < 2 * t.L ? swb : aswb);
      a.row0 = r0;
      a.nrows = std::min(rows_max, part_end - r0);
      r0 += a.nrows;
      a.nblobs = 1;
      a.n_groups = 1;
      a.groups[0].blob[0] = 0;
      for (int w = 1; w < 4; w++) a.groups[0].blob[w] = -1;
      a.prio = (size_t)a.nrows * t.nblk <= cap ? 1 : 0;
      EncBlob& B = a.b[0];
      init_enc_blob(B, t, chunks[i], qualities[i], outs_dev[i], caps[i]);
      size_t off = 64;
      B.lens = base + off;
      off = align64w(off + (size_t)a.nrows * t.C);
      B.row_words = base + off;
      off = align64w(off + (size_t)a.nrows);
      B.block_words = base + off;
      off = align64w(off + (size_t)a.nrows * t.nblk);
      B.scratch = base + off;
      B.status = status;
      HIP_TRY(launch_encode(a, st), "encode launch");
    }
    uint32_t sw[4];
    HIP_TRY(hipMemcpyAsync(sw, status, sizeof(sw), hipMemcpyDeviceToHost, st), "encode status");
    HIP_TRY(hipStreamSynchronize(st), "encode");
    finish_blob(t, chunks[i], sw, &out_lens[i], &rc);
  }
  return rc;
}

int cg_encode(const cg_tables* h, const void* k_dev, const void* v_dev, int32_t chunk,
              int32_t quality, void* out_dev, size_t cap, size_t* out_len, void* stream) {
  if (!out_len) return fail(CG_E_INVAL, "NULL argument");
  return cg_encode_batch(h, k_dev, v_dev, 1, &chunk, &quality, &out_dev, &cap, out_len, stream);
}

int cg_decode_async(const cg_tables* h, int32_t n, const void* const* blobs_dev,
                    const cg_chunk_info* infos, void* k_out_dev, void* v_out_dev,
                    uint32_t* status_dev, void* stream) {
  if (!h || n < 0 || (n > 0 && (!blobs_dev || !infos)) || !k_out_dev || !v_out_dev || !status_dev)
    return fail(CG_E_INVAL, "NULL argument");
  for (int i = 0; i < n; i++) {
    if (!blobs_dev[i]) return fail(CG_E_INVAL, "NULL blob");
    int rc = check_info_against(h, infos[i]);
    if (rc) return rc;
  }
  if (n == 0) return CG_OK;
  DeviceGuard dg(h->dev);
  if (!dg.ok) return fail(CG_E_HIP, "cannot select the tables' device");
  return enqueue_decode(h, n, blobs_dev, infos, k_out_dev, v_out_dev, status_dev,
                        static_cast<hipStream_t>(stream));
}

int cg_decode_paged_async(const cg_tables* h, int32_t n, const void* const* blobs_dev,
                          const cg_chunk_info* infos, void* k_pool_dev, void* v_pool_dev,
                          int64_t num_pages, int32_t page_tokens, const int32_t* block_table_dev,
                          int64_t n_blocks, uint32_t* status_dev, void* stream) {
  if (!h || n < 0 || (n > 0 && (!blobs_dev || !infos)) || !k_pool_dev || !v_pool_dev ||
      !status_dev || !block_table_dev)
    return fail(CG_E_INVAL, "NULL argument");
  const DevTables& t = h->t;
  if (page_tokens < 1 || page_tokens > kMaxChunk || (page_tokens & (page_tokens - 1)))
    return fail(CG_E_INVAL, "page_tokens must be a power of two in [1, 65536]");
  if (num_pages < 1 || num_pages > (int64_t)1 << 31 || n_blocks < 1 || n_blocks > (int64_t)1 << 30)
    return fail(CG_E_INVAL, "num_pages or n_blocks out of range");
  if ((uint64_t)num_pages * (uint64_t)page_tokens * (uint64_t)t.C * 2u >= (uint64_t)1 << 31)
    return fail(CG_E_INVAL, "a layer's pool must be smaller than 2 GiB");
  // lane j of a wave holds the row of token j of a group: every 64-channel
  // block needs at least a group's worth of channels
  const int last_blk = t.C - (t.nblk - 1) * 64;
  if (t.G > 64 || last_blk < t.G)
    return fail(CG_E_INVAL, "paged decode needs group_tokens <= 64 and at least group_tokens "
                            "channels in every 64-channel block");
  for (int i = 0; i < n; i++) {
    if (!blobs_dev[i]) return fail(CG_E_INVAL, "NULL blob");
    int rc = check_info_against(h, infos[i]);
    if (rc) return rc;
    const int64_t end = (int64_t)infos[i].token_offset + infos[i].chunk_tokens;
    if ((end + page_tokens - 1) / page_tokens > n_blocks)
      return fail(CG_E_INVAL, "block table shorter than the blobs' token ranges");
  }
  if (n == 0) return CG_OK;
  DeviceGuard dg(h->dev);
  if (!dg.ok) return fail(CG_E_HIP, "cannot select the tables' device");
  PagedOut pg;
  pg.table = block_table_dev;
  pg.n_blocks = (uint32_t)n_blocks;
  pg.num_pages = (uint32_t)num_pages;
  pg.shift = (uint32_t)__builtin_ctz((unsigned)page_tokens);
  return enqueue_decode(h, n, blobs_dev, infos, k_pool_dev, v_pool_dev, status_dev,
                        static_cast<hipStream_t>(stream), &pg);
}

int cg_decode(const cg_tables* ch, int32_t n, const void* const* blobs_dev, const size_t* lens,
              void* k_out_dev, void* v_out_dev, void* stream) {
  if (!ch || n < 0 || (n > 0 && (!blobs_dev || !lens)) || !k_out_dev || !v_out_dev)
    return fail(CG_E_INVAL, "NULL argument");
  cg_tables* h = const_cast<cg_tables*>(ch);
  DeviceGuard dg(h->dev);
  if (!dg.ok) return fail(CG_E_HIP, "cannot select the tables' device");
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<cg_chunk_info> infos(n);
  for (int i = 0; i < n; i++) {
    if (!blobs_dev[i]) return fail(CG_E_INVAL, "NULL blob");
    uint8_t hdr[kBlobHdr];
    if (lens[i] < (size_t)kBlobHdr) return fail(CG_E_INVAL, "blob shorter than its header");
    HIP_TRY(hipMemcpyAsync(hdr, blobs_dev[i], kBlobHdr, hipMemcpyDeviceToHost, st), "read header");
    HIP_TRY(hipStreamSynchronize(st), "read header");
    int rc = parse_info(hdr, kBlobHdr, &infos[i]);
    if (rc) return rc;
    if (infos[i].blob_bytes > lens[i]) return fail(CG_E_INVAL, "blob shorter than its header says");
    if ((rc = check_info_against(h, infos[i]))) return rc;
  }
  if (n == 0) return CG_OK;
  std::lock_guard<std::mutex> lk(h->mu);
  int rs = ensure_host_status(const_cast<cg_tables*>(h));  // a cache the lock guards
  if (rs) return rs;
  uint32_t* status = h->status + 8;
  HIP_TRY(hipMemsetAsync(status, 0, 4, st), "clear status");
  int rc = enqueue_decode(h, n, blobs_dev, infos.data(), k_out_dev, v_out_dev, status, st);
  if (rc) return rc;
  HIP_TRY(hipMemcpyAsync(h->host_status + 8, status, 4, hipMemcpyDeviceToHost, st), "status");
  HIP_TRY(hipStreamSynchronize(st), "decode");
  if (h->host_status[8]) return fail(CG_E_CORRUPT, "a blob failed validation while decoding");
  return CG_OK;
}

int cg_decode_streamed(const cg_tables* h, int32_t n, const void* const* blobs_host,
                       const cg_chunk_info* infos, void* k_out_dev, void* v_out_dev,
                       void* staging_dev, size_t staging_cap, uint32_t* status_dev,
                       void* copy_stream, void* compute_stream) {
  if (!h || n < 0 || (n > 0 && (!blobs_host || !infos)) || !k_out_dev || !v_out_dev ||
      !status_dev || !staging_dev)
    return fail(CG_E_INVAL, "NULL argument");
  size_t slot = 0;
  for (int i = 0; i < n; i++) {
    if (!blobs_host[i]) return fail(CG_E_INVAL, "NULL blob");
    int rc = check_info_against(h, infos[i]);
    if (rc) return rc;
    slot = std::max<size_t>(slot, (infos[i].blob_bytes + 255) & ~(size_t)255);
  }
  if (n == 0) return CG_OK;
  if (staging_cap < slot) return fail(CG_E_CAPACITY, "staging buffer smaller than a blob");
  const int nslots = (int)std::min<size_t>((size_t)n, staging_cap / slot);
  DeviceGuard dg(h->dev);
  if (!dg.ok) return fail(CG_E_HIP, "cannot select the tables' device");
  hipStream_t cs = static_cast<hipStream_t>(copy_stream);
  hipStream_t ks = static_cast<hipStream_t>(compute_stream);
  std::vector<hipEvent_t> copied(nslots, nullptr), done(nslots, nullptr);
  int rc = CG_OK;
  for (int s = 0; s < nslots && rc == CG_OK; s++) {
    if (hipEventCreateWithFlags(&copied[s], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&done[s], hipEventDisableTiming) != hipSuccess)
      rc = fail(CG_E_HIP, "event creation");
  }
  uint8_t* stage = static_cast<uint8_t*>(staging_dev);
  for (int i = 0; i < n && rc == CG_OK; i++) {
    const int s = i % nslots;
    uint8_t* dst = stage + (size_t)s * slot;
    hipError_t e = hipSuccess;
    if (i >= nslots) e = hipStreamWaitEvent(cs, done[s], 0);  // slot's last decode finished
    if (e == hipSuccess) e = hipMemcpyAsync(dst, blobs_host[i], infos[i].blob_bytes,
                                            hipMemcpyHostToDevice, cs);
    if (e == hipSuccess) e = hipEventRecord(copied[s], cs);
    if (e == hipSuccess) e = hipStreamWaitEvent(ks, copied[s], 0);
    if (e != hipSuccess) {
      rc = hip_fail(e, "pipeline copy");
      break;
    }
    const void* b = dst;
    rc = enqueue_decode(h, 1, &b, &infos[i], k_out_dev, v_out_dev, status_dev, ks);
    if (rc == CG_OK && (e = hipEventRecord(done[s], ks)) != hipSuccess)
      rc = hip_fail(e, "pipeline event");
  }
  for (int s = 0; s < nslots; s++) {
    if (copied[s]) (void)hipEventDestroy(copied[s]);
    if (done[s]) (void)hipEventDestroy(done[s]);
  }
  return rc;
}

}  // extern "C"

// Frees what the library keeps between calls on every device it has used:
// the table-build and encode workspaces, and the blocks its memory pool has
// cached but nothing holds.  A device's locks are taken in the order the other
// calls nest them (a build holds its workspace's lock while it allocates from
// the pool), then the device is waited for before anything is freed.
int cg_release_cached(void) {
  int rc = CG_OK;
  for (int dev = 0; dev < kMaxDevices; dev++) {
    BuildWs* b = build_ws(dev);
    EncWs* e = enc_ws(dev);
    KeepPool* kp = keep_pool_of(dev);
    std::unique_lock<std::mutex> lb(b->mu);
    std::unique_lock<std::mutex> le(e->mu);
    std::unique_lock<std::mutex> lp(kp->mu);
    if (!b->dev && !b->host && !e->scratch && !e->lens && !e->row_words && !e->status &&
        !e->host && !kp->pool)
      continue;
    DeviceGuard g(dev);
    if (!g.ok) {
      rc = fail(CG_E_HIP, "cannot select device " + std::to_string(dev));
      continue;
    }
    const hipError_t se = hipDeviceSynchronize();
    if (se != hipSuccess) {
      rc = hip_fail(se, "release: device synchronize");
      continue;
    }
    if (b->dev) (void)hipFree(b->dev);
    if (b->host) (void)hipHostFree(b->host);
    b->dev = nullptr;
    b->host = nullptr;
    b->bytes = 0;
    for (uint32_t** d : {&e->scratch, &e->lens, &e->row_words, &e->status})
      if (*d) {
        (void)hipFree(*d);
        *d = nullptr;
      }
    if (e->host) (void)hipHostFree(e->host);
    e->host = nullptr;
    e->scratch_bytes = e->lens_bytes = e->row_bytes = e->status_bytes = 0;
    if (kp->pool) {
      const hipError_t te = hipMemPoolTrimTo(kp->pool, 0);
      if (te != hipSuccess) rc = hip_fail(te, "release: pool trim");
    }
  }
  return rc;
}
