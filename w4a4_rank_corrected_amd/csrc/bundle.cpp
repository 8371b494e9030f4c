// Stored layer files: a prepared INT4 layer written to and read from disk
// ([Review] = "SVDQuant: How a Small High-Precision Branch Makes 4-Bit
// Diffusion Practical", sec. 5 Algorithm 1 step 9: the protected factors, the
// quantized residual, its scales and the smoothing transform are kept, so a
// layer is prepared once).
//
// File layout (little-endian), version 1:
//   header, 64 bytes:
//     char     magic[8]      "SVDQLAYR"
//     uint32   version       1
//     uint32   format        0 = INT4 codes, group 64, fp16 scales
//     int32    m, n, rank, group
//     float    alpha         migration strength the layer was prepared with
//     uint32   flags         bit 0: a bias is stored
//     uint64   payload_bytes
//     uint64   checksum      FNV-1a (64-bit) of the payload bytes
//     uint8    reserved[8]   zero
//   payload, in this order, each array contiguous:
//     lambda fp32 [m], smooth_inv fp32 [m], qw [m/64][n][32], wscale fp16
//     [m/64][n], l1 bf16 [rank][m], l2 bf16 [n][rank], bias bf16 [n] (flag)
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

using namespace svdq;

namespace {

constexpr char kMagic[8] = {'S', 'V', 'D', 'Q', 'L', 'A', 'Y', 'R'};
constexpr uint32_t kVersion = 1;
constexpr uint32_t kFormatInt4 = 0;

struct Header {
  char magic[8];
  uint32_t version, format;
  int32_t m, n, rank, group;
  float alpha;
  uint32_t flags;
  uint64_t payload_bytes, checksum;
  uint8_t reserved[8];
};
static_assert(sizeof(Header) == 64, "64-byte header");

uint64_t fnv1a(const uint8_t* p, size_t len, uint64_t h = 0xCBF29CE484222325ull) {
  for (size_t i = 0; i < len; ++i) {
    h ^= p[i];
    h *= 0x100000001B3ull;
  }
  return h;
}

struct Part {
  const void* src;
  void* dst;
  size_t bytes;
};

// the payload arrays of a layer of these dimensions, in file order
std::vector<size_t> part_sizes(int m, int n, int rank, bool bias) {
  const size_t G = (size_t)m / SVDQ_GROUP;
  std::vector<size_t> s = {4 * (size_t)m, 4 * (size_t)m, G * (size_t)n * 32, 2 * G * (size_t)n,
                           2 * (size_t)rank * m, 2 * (size_t)n * rank};
  if (bias) s.push_back(2 * (size_t)n);
  return s;
}

int check_dims(int m, int n, int rank, int group) {
  if (group != SVDQ_GROUP || m < SVDQ_GROUP || m % SVDQ_GROUP || m > SVDQ_MAX_DIM) {
    set_error("layer file: m must be a positive multiple of 64 up to %d and group 64 (got m=%d group=%d)",
              SVDQ_MAX_DIM, m, group);
    return SVDQ_ERR_UNSUPPORTED;
  }
  if (n < 1 || n > SVDQ_MAX_DIM || rank < 0 || rank > SVDQ_MAX_RANK || rank > (m < n ? m : n)) {
    set_error("layer file: bad n=%d or rank=%d", n, rank);
    return SVDQ_ERR_INVALID_ARG;
  }
  return SVDQ_OK;
}

// Reads and validates the header of an open file; leaves the position after it.
int read_header(FILE* f, const char* path, Header& h) {
  if (std::fread(&h, sizeof h, 1, f) != 1) {
    set_error("layer file %s: cannot read the 64-byte header", path);
    return SVDQ_ERR_IO;
  }
  if (std::memcmp(h.magic, kMagic, 8) != 0) {
    set_error("layer file %s: not a layer file (bad magic)", path);
    return SVDQ_ERR_IO;
  }
  if (h.version != kVersion || h.format != kFormatInt4) {
    set_error("layer file %s: version %u format %u not supported (this library reads version %u format %u)",
              path, h.version, h.format, kVersion, kFormatInt4);
    return SVDQ_ERR_IO;
  }
  const int st = check_dims(h.m, h.n, h.rank, h.group);
  if (st) return st;
  size_t total = 0;
  for (size_t s : part_sizes(h.m, h.n, h.rank, h.flags & 1u)) total += s;
  if (h.payload_bytes != total) {
    set_error("layer file %s: payload of %llu bytes, %zu expected for m=%d n=%d rank=%d", path,
              (unsigned long long)h.payload_bytes, total, h.m, h.n, h.rank);
    return SVDQ_ERR_IO;
  }
  return SVDQ_OK;
}

}  // namespace

extern "C" {

int svdq_save_layer(const char* path, const svdq_host_layer* L) {
  clear_error();
  if (!path || !L) {
    set_error("path and layer must not be NULL");
    return SVDQ_ERR_INVALID_ARG;
  }
  int st = check_dims(L->m, L->n, L->rank, L->group);
  if (st) return st;
  if (!L->lambda || !L->smooth_inv || !L->qw || !L->wscale || (L->rank > 0 && (!L->l1 || !L->l2))) {
    set_error("layer arrays lambda, smooth_inv, qw, wscale (and l1, l2 when rank > 0) must not be NULL");
    return SVDQ_ERR_INVALID_ARG;
  }
  const bool bias = L->bias != nullptr;
  const std::vector<size_t> sizes = part_sizes(L->m, L->n, L->rank, bias);
  const void* src[7] = {L->lambda, L->smooth_inv, L->qw, L->wscale, L->l1, L->l2, L->bias};
  Header h{};
  std::memcpy(h.magic, kMagic, 8);
  h.version = kVersion;
  h.format = kFormatInt4;
  h.m = L->m;
  h.n = L->n;
  h.rank = L->rank;
  h.group = L->group;
  h.alpha = L->alpha;
  h.flags = bias ? 1u : 0u;
  uint64_t sum = 0xCBF29CE484222325ull;
  for (size_t i = 0; i < sizes.size(); ++i) {
    h.payload_bytes += sizes[i];
    if (sizes[i]) sum = fnv1a(static_cast<const uint8_t*>(src[i]), sizes[i], sum);
  }
  h.checksum = sum;
  // write to a temporary name, then rename: a reader never sees a partial file
  const std::string tmp = std::string(path) + ".tmp";
  FILE* f = std::fopen(tmp.c_str(), "wb");
  if (!f) {
    set_error("cannot open %s for writing", tmp.c_str());
    return SVDQ_ERR_IO;
  }
  bool ok = std::fwrite(&h, sizeof h, 1, f) == 1;
  for (size_t i = 0; ok && i < sizes.size(); ++i)
    ok = sizes[i] == 0 || std::fwrite(src[i], 1, sizes[i], f) == sizes[i];
  ok = (std::fclose(f) == 0) && ok;
  if (!ok || std::rename(tmp.c_str(), path) != 0) {
    std::remove(tmp.c_str());
    set_error("writing %s failed", path);
    return SVDQ_ERR_IO;
  }
  return SVDQ_OK;
}

int svdq_load_layer_info(const char* path, int32_t* m, int32_t* n, int32_t* rank, int32_t* has_bias,
                         float* alpha) {
  clear_error();
  if (!path || !m || !n || !rank || !has_bias) {
    set_error("path, m, n, rank and has_bias must not be NULL");
    return SVDQ_ERR_INVALID_ARG;
  }
  FILE* f = std::fopen(path, "rb");
  if (!f) {
    set_error("cannot open %s", path);
    return SVDQ_ERR_IO;
  }
  Header h;
  const int st = read_header(f, path, h);
  std::fclose(f);
  if (st) return st;
  *m = h.m;
  *n = h.n;
  *rank = h.rank;
  *has_bias = (int32_t)(h.flags & 1u);
  if (alpha) *alpha = h.alpha;
  return SVDQ_OK;
}

int svdq_load_layer(const char* path, float* lambda, float* smooth_inv, uint8_t* qw, uint16_t* wscale,
                    uint16_t* l1, uint16_t* l2, uint16_t* bias) {
  clear_error();
  if (!path || !lambda || !smooth_inv || !qw || !wscale) {
    set_error("path, lambda, smooth_inv, qw and wscale must not be NULL");
    return SVDQ_ERR_INVALID_ARG;
  }
  FILE* f = std::fopen(path, "rb");
  if (!f) {
    set_error("cannot open %s", path);
    return SVDQ_ERR_IO;
  }
  Header h;
  int st = read_header(f, path, h);
  if (st) {
    std::fclose(f);
    return st;
  }
  const bool has_bias = h.flags & 1u;
  if ((h.rank > 0 && (!l1 || !l2)) || (has_bias && !bias)) {
    std::fclose(f);
    set_error("l1 and l2 (rank %d) and bias (stored: %d) must not be NULL", h.rank, (int)has_bias);
    return SVDQ_ERR_INVALID_ARG;
  }
  // read into host staging first: the caller's buffers are written only when
  // the whole payload is present and its checksum matches
  const std::vector<size_t> sizes = part_sizes(h.m, h.n, h.rank, has_bias);
  std::vector<uint8_t> buf(h.payload_bytes);
  const bool got = buf.empty() || std::fread(buf.data(), 1, buf.size(), f) == buf.size();
  const bool trailing = std::fgetc(f) != EOF;
  std::fclose(f);
  if (!got || trailing) {
    set_error("layer file %s: payload %s", path, got ? "followed by extra bytes" : "truncated");
    return SVDQ_ERR_IO;
  }
  if (fnv1a(buf.data(), buf.size()) != h.checksum) {
    set_error("layer file %s: checksum mismatch (corrupted file)", path);
    return SVDQ_ERR_IO;
  }
  void* dst[7] = {lambda, smooth_inv, qw, wscale, l1, l2, bias};
  size_t off = 0;
  for (size_t i = 0; i < sizes.size(); ++i) {
    if (sizes[i]) std::memcpy(dst[i], buf.data() + off, sizes[i]);
    off += sizes[i];
  }
  return SVDQ_OK;
}

}  // extern "C"
