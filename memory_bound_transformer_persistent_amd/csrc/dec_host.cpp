// Host runtime behind include/dec.h: model-description checks, DECW weight
// file ingest, the host packer, the device arena, and the launches of the
// resident decode kernel (dec_kernels.hip).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/dec.h"
#include "dec_internal.h"

using namespace decmono;

namespace {

thread_local std::string g_err;   // last error of a handle-less call on this thread

int fail(std::string* where, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  (where ? *where : g_err) = buf;
  return code;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t n, size_t a = kAlign) { return (n + a - 1) / a * a; }

bool moe(const dec_model_desc& d) { return d.n_experts > 0; }
bool mxfp4(const dec_model_desc& d) { return moe(d) && (d.flags & DEC_FLAG_EXPERTS_MXFP4) != 0; }
// canonical tensors per layer: dense 9; mixture of experts 13 (the MLP's
// three matrices become the router, three code matrices and their scales)
int per_layer(const dec_model_desc& d) { return moe(d) ? 13 : 9; }
int n_tensors_for(const dec_model_desc& d) { return 1 + per_layer(d) * d.n_layers + 2; }
// which resident kernel runs the model: its batch, or the mixture-of-experts one
int kernel_kind(const dec_model_desc& d) { return moe(d) ? kMoeKernel : d.batch; }

int check_desc_impl(const dec_model_desc* d, std::string* err) {
  if (!d) return fail(err, DEC_ERR_INVALID_ARG, "model description is NULL");
  if (d->n_layers < 1) return fail(err, DEC_ERR_BAD_DESC, "n_layers must be >= 1 (got %d)", d->n_layers);
  if (d->d_model < 8 || d->d_model % 8) return fail(err, DEC_ERR_BAD_DESC, "d_model must be a positive multiple of 8 (got %d)", d->d_model);
  if (d->n_heads < 1) return fail(err, DEC_ERR_BAD_DESC, "n_heads must be >= 1 (got %d)", d->n_heads);
  if (d->n_kv_heads != d->n_heads) return fail(err, DEC_ERR_BAD_DESC, "n_kv_heads must equal n_heads (multi-head attention)");
  const int hd = d->head_dim;
  if (hd != 8 && hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return fail(err, DEC_ERR_BAD_DESC, "head_dim must be one of 8,16,32,64,128 (got %d)", hd);
  if (d->d_ffn < 8 || d->d_ffn % 8) return fail(err, DEC_ERR_BAD_DESC, "d_ffn must be a positive multiple of 8 (got %d)", d->d_ffn);
  if (d->vocab < 1) return fail(err, DEC_ERR_BAD_DESC, "vocab must be >= 1");
  if (d->lm_vocab < 2 || d->lm_vocab > d->vocab || d->lm_vocab % 2)
    return fail(err, DEC_ERR_BAD_DESC, "lm_vocab must be even and in [2, vocab] (got %d)", d->lm_vocab);
  if (d->max_ctx < 1 || d->max_ctx > 65536) return fail(err, DEC_ERR_BAD_DESC, "max_ctx must be in [1, 65536] (got %d)", d->max_ctx);
  if (!(d->rms_eps > 0.f) || !std::isfinite(d->rms_eps)) return fail(err, DEC_ERR_BAD_DESC, "rms_eps must be > 0");
  if (!(d->rope_base > 1.f) || !std::isfinite(d->rope_base)) return fail(err, DEC_ERR_BAD_DESC, "rope_base must be > 1");
  if (d->flags & ~(DEC_FLAG_BATCHED_PREFILL | DEC_FLAG_MATRIX_PREFILL | DEC_FLAG_EXPERTS_MXFP4))
    return fail(err, DEC_ERR_BAD_DESC, "unknown flags 0x%x", d->flags);
  if ((d->flags & DEC_FLAG_EXPERTS_MXFP4) && d->n_experts == 0)
    return fail(err, DEC_ERR_BAD_DESC, "DEC_FLAG_EXPERTS_MXFP4 is for a mixture of experts");
  const bool bp = (d->flags & DEC_FLAG_BATCHED_PREFILL) != 0;
  const bool mp = (d->flags & DEC_FLAG_MATRIX_PREFILL) != 0;
  if (bp && mp) return fail(err, DEC_ERR_BAD_DESC, "DEC_FLAG_BATCHED_PREFILL and DEC_FLAG_MATRIX_PREFILL exclude each other");
  if (bp && d->batch != 1) return fail(err, DEC_ERR_BAD_DESC, "DEC_FLAG_BATCHED_PREFILL is for batch 1");
  if (mp && d->batch != 1) return fail(err, DEC_ERR_BAD_DESC, "DEC_FLAG_MATRIX_PREFILL is for batch 1");
  if (d->batch < 1) return fail(err, DEC_ERR_BAD_DESC, "batch must be >= 1");
  if (d->n_experts == 0) {
    if (d->top_k != 0) return fail(err, DEC_ERR_BAD_DESC, "top_k must be 0 for a dense model (got %d)", d->top_k);
  } else {
    if (d->n_experts < 2 || d->n_experts > kMoeMaxExperts || d->n_experts % 2)
      return fail(err, DEC_ERR_BAD_DESC, "n_experts must be 0 or even and in [2, %d] (got %d)", kMoeMaxExperts, d->n_experts);
    if (d->top_k < 1 || d->top_k > std::min(d->n_experts, kMoeMaxTopK))
      return fail(err, DEC_ERR_BAD_DESC, "top_k must be in [1, min(n_experts, %d)] (got %d)", kMoeMaxTopK, d->top_k);
    if (d->batch != 1 || (d->flags & ~DEC_FLAG_EXPERTS_MXFP4))
      return fail(err, DEC_ERR_UNSUPPORTED, "a mixture-of-experts model runs at batch 1 with flags 0 or "
                  "DEC_FLAG_EXPERTS_MXFP4");
    if (d->d_model % 16 || d->d_ffn % 16)
      return fail(err, DEC_ERR_UNSUPPORTED, "a mixture-of-experts model needs d_model and d_ffn multiples of 16");
    if ((d->flags & DEC_FLAG_EXPERTS_MXFP4) && (d->d_model % 32 || d->d_ffn % 32))
      return fail(err, DEC_ERR_UNSUPPORTED, "MXFP4 experts need d_model and d_ffn multiples of 32");
    if ((long long)d->top_k * d->d_ffn > kMaxK - 1024)
      return fail(err, DEC_ERR_UNSUPPORTED, "top_k * d_ffn must be <= %d", kMaxK - 1024);
    if ((long long)d->n_experts * 2 * d->d_ffn * d->d_model >= (1LL << 31))
      return fail(err, DEC_ERR_UNSUPPORTED, "a layer's expert codes must be under 2 GiB");
  }
  const long long q = (long long)d->n_heads * hd;
  if (q % 8) return fail(err, DEC_ERR_BAD_DESC, "n_heads*head_dim must be a multiple of 8");
  if (mp && (hd < 32 || d->d_model % 32 || q % 32 || d->d_ffn % 32))
    return fail(err, DEC_ERR_UNSUPPORTED, "DEC_FLAG_MATRIX_PREFILL needs head_dim >= 32 and d_model, "
                "n_heads*head_dim, d_ffn multiples of 32");
  if (d->batch > kMaxBatch) return fail(err, DEC_ERR_UNSUPPORTED, "batch must be <= %d", kMaxBatch);
  if (d->batch > 1 || bp) {
    auto span = [](long long k) { return (k + 511) / 512 * 512; };
    if (span(d->d_model) > kBatchSpanD || span(d->d_ffn) > kBatchSpanK || span(q) > kBatchSpanK)
      return fail(err, DEC_ERR_UNSUPPORTED,
                  "batch > 1 needs d_model <= %d and d_ffn, n_heads*head_dim <= %d (inputs kept in LDS)",
                  kBatchSpanD, kBatchSpanK);
  }
  if (d->d_model > kMaxK || q > kMaxK || d->d_ffn > kMaxK)
    return fail(err, DEC_ERR_UNSUPPORTED, "d_model, n_heads*head_dim and d_ffn must be <= %d", kMaxK);
  // largest matrix must be addressable with 32-bit byte offsets
  const long long lm_bytes = 2LL * d->lm_vocab * d->d_model;
  const long long big = std::max({lm_bytes, 2LL * 3 * q * d->d_model, 2LL * 2 * d->d_ffn * d->d_model});
  if (big >= (1LL << 31)) return fail(err, DEC_ERR_UNSUPPORTED, "a weight matrix is 2 GiB or larger");
  if (2LL * d->max_ctx * hd >= (1LL << 31)) return fail(err, DEC_ERR_UNSUPPORTED, "KV cache of one head is 2 GiB or larger");
  const int hb = (bp ? kMaxBatch : d->batch) * d->n_heads;
  if (hb > kMaxHeads) return fail(err, DEC_ERR_UNSUPPORTED, "batch (8 with batched prefill) x n_heads must be <= %d",
                                  kMaxHeads);
  if ((long long)hb * max_attn_chunks(d->max_ctx, hb, 1024) > 65536)
    return fail(err, DEC_ERR_UNSUPPORTED, "too many attention partials (batch x n_heads x chunks > 65536)");
  return DEC_OK;
}

// ---------------------------------------------------------------------------
// packed image layout (elements)
// ---------------------------------------------------------------------------
// Batch 1: every matrix row-major.  Batch > 1: every GEMV matrix (not the
// embedding) in tiles of 16 rows x 32 columns, one 1 KB tile per MFMA
// operand (see tiled_index).
// Mixture of experts: the fp16 image holds the router where the dense
// model's Wgu is (off_gu, [E, d]) and no Wd; the experts live in an image of
// their own (bytes): per layer Wgu8 [E][F][2][d] (gate row j and up row j of
// expert e at rows 2(eF + j), 2(eF + j) + 1), then Wd8 [E][d][F]; and their
// row scales (floats): per layer [E][F][2] (gate, up), then [E][d].
struct Image {
  size_t off_qkv, off_o, off_gu, off_d, layer_stride, off_E, off_lm, total;
  bool tiled;
  size_t e8_d, e8_stride, e8_total;     // expert codes (bytes)
  size_t sc_d, sc_stride, sc_total;     // expert row scales (floats), or MXFP4 block scales (bytes)
};

size_t al128(size_t n) { return (n + 127) / 128 * 128; }

// elements a [rows x cols] matrix occupies in the image
size_t matrix_elems(size_t rows, size_t cols, bool tiled) {
  if (!tiled) return rows * cols;
  return ((rows + kTileRows - 1) / kTileRows) * ((cols + kTileCols - 1) / kTileCols) * kTileElems;
}

// Tiled layout: tile (g, j) covers rows 16g..16g+15 and columns 32j..32j+31
// and sits at tile index g * ceil(cols/32) + j.  Inside a tile, lane l's 8
// elements (16 bytes at 16 l) are row 16g + l % 16, columns 32j + 8 (l / 16)
// .. +7: the A operand of v_mfma_f32_16x16x32_f16 for a wave that loads the
// tile with one 16-byte load per lane.  Padding rows and columns are zero.
size_t tiled_index(size_t r, size_t c, size_t cols) {
  const size_t kt = (cols + kTileCols - 1) / kTileCols;
  const size_t tile = (r / kTileRows) * kt + c / kTileCols;
  const size_t lane = (r % kTileRows) + kTileRows * ((c % kTileCols) / 8);
  return tile * kTileElems + lane * 8 + c % 8;
}

Image image_layout(const dec_model_desc& d) {
  Image im;
  const size_t D = d.d_model, q = (size_t)d.n_heads * d.head_dim, F = d.d_ffn;
  const bool t = d.batch > 1;
  im.tiled = t;
  im.off_qkv = 0;
  im.off_o = al128(im.off_qkv + matrix_elems(3 * q, D, t));
  im.off_gu = al128(im.off_o + matrix_elems(D, q, t));
  im.e8_d = im.e8_stride = im.e8_total = im.sc_d = im.sc_stride = im.sc_total = 0;
  if (moe(d)) {
    const size_t E = d.n_experts;
    im.off_d = al128(im.off_gu + E * D);
    im.layer_stride = im.off_d;
    if (mxfp4(d)) {
      // E2M1 pairs: half a byte per weight; E8M0 scales: a byte per 32 weights
      im.e8_d = align_up(E * F * D);
      im.e8_stride = align_up(im.e8_d + E * D * F / 2);
      im.sc_d = E * F * 2 * (D / 32);
      im.sc_stride = align_up(im.sc_d + E * D * (F / 32));
    } else {
      im.e8_d = align_up(E * 2 * F * D);
      im.e8_stride = align_up(im.e8_d + E * D * F);
      im.sc_d = E * F * 2;
      im.sc_stride = align_up(im.sc_d + E * D, 64);
    }
    im.e8_total = im.e8_stride * d.n_layers;
    im.sc_total = im.sc_stride * d.n_layers;
  } else {
    im.off_d = al128(im.off_gu + matrix_elems(2 * F, D, t));
    im.layer_stride = al128(im.off_d + matrix_elems(D, F, t));
  }
  im.off_E = im.layer_stride * d.n_layers;
  im.off_lm = al128(im.off_E + (size_t)d.vocab * D);
  im.total = al128(im.off_lm + matrix_elems(d.lm_vocab, D, t));
  return im;
}

// Row `row` (C elements) of a packed matrix with `cols` columns starting at
// element `base`: copied as it is (row-major) or scattered into tiles.
void put_row(uint16_t* image, size_t base, size_t row, const uint16_t* src, size_t cols, bool tiled) {
  if (!tiled) {
    std::memcpy(image + base + row * cols, src, cols * 2);
    return;
  }
  for (size_t c = 0; c < cols; c += 8) std::memcpy(image + base + tiled_index(row, c, cols), src + c, 16);
}

// shape of canonical tensor `idx`
void tensor_shape(const dec_model_desc& d, int idx, size_t* r, size_t* c) {
  const size_t D = d.d_model, q = (size_t)d.n_heads * d.head_dim, F = d.d_ffn;
  const int last = n_tensors_for(d) - 1;
  if (idx == 0) { *r = d.vocab; *c = D; return; }
  if (idx == last) { *r = d.lm_vocab; *c = D; return; }
  if (idx == last - 1) { *r = D; *c = 1; return; }
  if (moe(d)) {
    const size_t E = d.n_experts;
    const bool mx = mxfp4(d);
    switch ((idx - 1) % 13) {
      case 0: case 5: *r = D; *c = 1; return;            // gains
      case 1: case 2: case 3: *r = q; *c = D; return;     // Wq, Wk, Wv
      case 4: *r = D; *c = q; return;                     // Wo
      case 6: *r = E; *c = D; return;                     // Wr
      case 7: case 9: *r = E * F; *c = mx ? D / 2 : D; return;     // Wg8, Wu8 (MXFP4: code pairs)
      case 8: case 10: *r = E * F; *c = mx ? D / 32 : 1; return;   // sg, su (MXFP4: block scales)
      case 11: *r = E * D; *c = mx ? F / 2 : F; return;            // Wd8
      default: *r = E * D; *c = mx ? F / 32 : 1; return;           // sd
    }
  }
  switch ((idx - 1) % 9) {
    case 0: case 5: *r = D; *c = 1; return;            // gains
    case 1: case 2: case 3: *r = q; *c = D; return;     // Wq, Wk, Wv
    case 4: *r = D; *c = q; return;                     // Wo
    case 6: case 7: *r = F; *c = D; return;             // Wg, Wu
    default: *r = D; *c = F; return;                   // Wd
  }
}

// Place canonical tensor idx (row-major) into the packed image; gains go to
// gains_out (fp32) instead, expert codes to image8 and their scales to
// scales (a mixture of experts).  Rows may be passed in slices.
void place_tensor(const dec_model_desc& d, const Image& im, int idx, const uint16_t* src,
                  size_t row0, size_t nrows, uint16_t* image, float* gains_out, uint8_t* image8 = nullptr,
                  float* scales = nullptr) {
  size_t R, C;
  tensor_shape(d, idx, &R, &C);
  const size_t D = d.d_model, q = (size_t)d.n_heads * d.head_dim;
  const int last = n_tensors_for(d) - 1;
  auto half_to_float = [](uint16_t h) {
    const uint32_t s = (uint32_t)(h >> 15) << 31;
    const uint32_t e = (h >> 10) & 0x1f, m = h & 0x3ff;
    uint32_t bits;
    if (e == 0) {
      if (m == 0) bits = s;
      else {  // subnormal: value m * 2^-24, exact in fp32
        float f = (float)m * 5.9604644775390625e-08f;
        std::memcpy(&bits, &f, 4);
        bits |= s;
      }
    } else if (e == 31) bits = s | 0x7f800000u | (m << 13);
    else bits = s | ((e + 112) << 23) | (m << 13);
    float f;
    std::memcpy(&f, &bits, 4);
    return f;
  };
  if (idx == 0) {
    std::memcpy(image + im.off_E + row0 * C, src, nrows * C * 2);
    return;
  }
  if (idx == last) {
    for (size_t i = 0; i < nrows; ++i) put_row(image, im.off_lm, row0 + i, src + i * C, C, im.tiled);
    return;
  }
  if (idx == last - 1) {
    for (size_t i = 0; i < nrows; ++i) gains_out[(size_t)d.n_layers * 2 * D + row0 + i] = half_to_float(src[i]);
    return;
  }
  const int per = per_layer(d);
  const int l = (idx - 1) / per, kind = (idx - 1) % per;
  uint16_t* lay = image + (size_t)l * im.layer_stride;
  if (moe(d) && kind >= 6) {
    const size_t F = d.d_ffn;
    const uint8_t* s8 = reinterpret_cast<const uint8_t*>(src);
    const float* sf = reinterpret_cast<const float*>(src);
    uint8_t* lay8 = image8 + (size_t)l * im.e8_stride;
    float* lsc = scales + (size_t)l * im.sc_stride;
    // MXFP4: the scale image holds bytes (E8M0), C of them per row
    uint8_t* lsx = reinterpret_cast<uint8_t*>(scales) + (size_t)l * im.sc_stride;
    const bool mx = mxfp4(d);
    for (size_t i = 0; i < nrows; ++i) {
      const size_t r = row0 + i;
      switch (kind) {
        case 6: put_row(lay, im.off_gu, r, src + i * C, C, false); break;   // router
        case 7: case 9: std::memcpy(lay8 + (2 * r + (kind == 9)) * C, s8 + i * C, C); break;
        case 8: case 10:
          if (mx) std::memcpy(lsx + (2 * r + (kind == 10)) * C, s8 + i * C, C);
          else lsc[2 * r + (kind == 10)] = sf[i];
          break;
        case 11: std::memcpy(lay8 + im.e8_d + r * C, s8 + i * C, C); break;
        default:
          if (mx) std::memcpy(lsx + im.sc_d + r * C, s8 + i * C, C);
          else lsc[im.sc_d + r] = sf[i];
          break;
      }
    }
    return;
  }
  switch (kind) {
    case 0:
    case 5:
      for (size_t i = 0; i < nrows; ++i)
        gains_out[((size_t)l * 2 + (kind == 5)) * D + row0 + i] = half_to_float(src[i]);
      return;
    case 1: case 2: case 3:  // Wq, Wk, Wv stacked into Wqkv
      for (size_t i = 0; i < nrows; ++i) put_row(lay, im.off_qkv, (kind - 1) * q + row0 + i, src + i * C, C, im.tiled);
      return;
    case 4:
      for (size_t i = 0; i < nrows; ++i) put_row(lay, im.off_o, row0 + i, src + i * C, C, im.tiled);
      return;
    case 6: case 7:          // Wg -> even rows, Wu -> odd rows of Wgu
      for (size_t i = 0; i < nrows; ++i) put_row(lay, im.off_gu, 2 * (row0 + i) + (kind == 7), src + i * C, C, im.tiled);
      return;
    default:
      for (size_t i = 0; i < nrows; ++i) put_row(lay, im.off_d, row0 + i, src + i * C, C, im.tiled);
      return;
  }
}

// ---------------------------------------------------------------------------
// DECW weight file
// ---------------------------------------------------------------------------
constexpr size_t kHdrBytes = 72, kEntryBytes = 40;

struct FileEntry { uint32_t index, dtype, ndim, dim0, dim1; uint64_t offset, nbytes; };

template <class T> T rd(const unsigned char* p) { T v; std::memcpy(&v, p, sizeof v); return v; }

int read_file_header(FILE* f, dec_model_desc* out, std::vector<FileEntry>* entries, std::string* err) {
  unsigned char h[kHdrBytes];
  if (fseek(f, 0, SEEK_END) != 0) return fail(err, DEC_ERR_WEIGHTS, "cannot seek weight file");
  const long long fsize = ftell(f);
  fseek(f, 0, SEEK_SET);
  if (fsize < (long long)kHdrBytes || fread(h, 1, kHdrBytes, f) != kHdrBytes)
    return fail(err, DEC_ERR_WEIGHTS, "weight file shorter than its header");
  if (std::memcmp(h, "DECW", 4) != 0) return fail(err, DEC_ERR_WEIGHTS, "bad magic (not a DECW file)");
  if (rd<uint32_t>(h + 4) != 1) return fail(err, DEC_ERR_WEIGHTS, "unsupported DECW version %u", rd<uint32_t>(h + 4));
  const uint32_t n = rd<uint32_t>(h + 8);
  dec_model_desc d;
  std::memset(&d, 0, sizeof d);
  int32_t* ints = &d.n_layers;
  for (int i = 0; i < 10; ++i) ints[i] = rd<int32_t>(h + 16 + 4 * i);
  d.rms_eps = rd<float>(h + 56);
  d.rope_base = rd<float>(h + 60);
  d.flags = rd<uint32_t>(h + 64);
  int rc = check_desc_impl(&d, err);
  if (rc == DEC_ERR_BAD_DESC) return fail(err, DEC_ERR_WEIGHTS, "weight file description invalid: %s", err ? err->c_str() : g_err.c_str());
  if ((int)n != n_tensors_for(d)) return fail(err, DEC_ERR_WEIGHTS, "weight file has %u tensors, description needs %d", n, n_tensors_for(d));
  if (fsize < (long long)(kHdrBytes + n * kEntryBytes)) return fail(err, DEC_ERR_WEIGHTS, "weight file truncated in its tensor table");
  std::vector<unsigned char> tab(n * kEntryBytes);
  if (fread(tab.data(), 1, tab.size(), f) != tab.size()) return fail(err, DEC_ERR_WEIGHTS, "cannot read tensor table");
  entries->resize(n);
  for (uint32_t i = 0; i < n; ++i) {
    const unsigned char* e = tab.data() + i * kEntryBytes;
    FileEntry fe{rd<uint32_t>(e), rd<uint32_t>(e + 4), rd<uint32_t>(e + 8), rd<uint32_t>(e + 16), rd<uint32_t>(e + 20),
                 rd<uint64_t>(e + 24), rd<uint64_t>(e + 32)};
    size_t R, C;
    tensor_shape(d, (int)i, &R, &C);
    if (fe.index != i) return fail(err, DEC_ERR_WEIGHTS, "tensor %u: index field %u out of order", i, fe.index);
    if (fe.dtype != 1) return fail(err, DEC_ERR_WEIGHTS, "tensor %u: dtype %u is not fp16", i, fe.dtype);
    const bool vec = (C == 1);
    if (vec ? !(fe.ndim == 1 && fe.dim0 == R && fe.dim1 == 1) : !(fe.ndim == 2 && fe.dim0 == R && fe.dim1 == C))
      return fail(err, DEC_ERR_WEIGHTS, "tensor %u: shape (%u,%u) does not match the description (%zu,%zu)", i, fe.dim0, fe.dim1, R, C);
    if (fe.nbytes != 2ull * R * C) return fail(err, DEC_ERR_WEIGHTS, "tensor %u: nbytes %llu != %llu", i, (unsigned long long)fe.nbytes, 2ull * R * C);
    if (fe.offset % 256) return fail(err, DEC_ERR_WEIGHTS, "tensor %u: offset not 256-byte aligned", i);
    if (fe.offset < kHdrBytes + n * kEntryBytes || fe.offset + fe.nbytes > (uint64_t)fsize)
      return fail(err, DEC_ERR_WEIGHTS, "tensor %u: payload [%llu, %llu) outside the file (size %lld)", i,
                  (unsigned long long)fe.offset, (unsigned long long)(fe.offset + fe.nbytes), fsize);
    (*entries)[i] = fe;
  }
  *out = d;
  return DEC_OK;
}

bool same_shape(const dec_model_desc& a, const dec_model_desc& b) {
  return a.n_layers == b.n_layers && a.d_model == b.d_model && a.n_heads == b.n_heads && a.n_kv_heads == b.n_kv_heads &&
         a.head_dim == b.head_dim && a.d_ffn == b.d_ffn && a.vocab == b.vocab && a.lm_vocab == b.lm_vocab &&
         a.n_experts == b.n_experts && a.top_k == b.top_k;
}

// ---------------------------------------------------------------------------
// device arena layout (bytes)
// ---------------------------------------------------------------------------
struct Arena {
  size_t w, w2, w8, esc, routes, rpart, gains, rope, kv, mp_x, mp_h, mp_q16, mp_a, mp_s, mp_part, x, xg16, ssp, qkv, att_o, part, pml, act, logits, amax_v, amax_i, tok_cur, tok_out,
      prompt, ctl, srv_slot, params, params2, trace, total;
};

bool batched_prefill(const dec_model_desc& d) { return (d.flags & DEC_FLAG_BATCHED_PREFILL) != 0; }
bool matrix_prefill(const dec_model_desc& d) { return (d.flags & DEC_FLAG_MATRIX_PREFILL) != 0; }

// The matrix prefill's workspace: prompt positions per pass over the
// weights, and the floats of its split-K partial sums.
int mp_chunk(const dec_model_desc& d) { return std::min(d.max_ctx, kMpChunk); }
size_t mp_part_floats(const dec_model_desc& d) {
  const size_t q = (size_t)d.n_heads * d.head_dim;
  const size_t widest = std::max({3 * q, 2 * (size_t)d.d_ffn, (size_t)d.d_model});
  return std::min(kMpPartFloats, 8 * std::max((size_t)mp_chunk(d) * widest, (size_t)d.lm_vocab));
}

// The description the batched prefill kernel runs with: kMaxBatch columns
// (consecutive positions of the one sequence) and the tiled weight image.
dec_model_desc prefill_desc(const dec_model_desc& d) {
  dec_model_desc p = d;
  p.batch = kMaxBatch;
  p.flags = 0;
  return p;
}

Arena arena_layout(const dec_model_desc& d, int G) {
  Arena a;
  const Image im = image_layout(d);
  a.rpart = 0;
  const size_t D = d.d_model, q = (size_t)d.n_heads * d.head_dim;
  const bool bp = batched_prefill(d);
  // rows of the per-column buffers: sequences, or the batched prefill's columns
  const size_t B = bp ? (size_t)kMaxBatch : (size_t)d.batch;
  const size_t hb = B * d.n_heads;   // attention heads of all columns
  const size_t hkv = (size_t)d.batch * d.n_heads;   // heads with a KV cache
  const size_t part_rows = std::max(hkv * max_attn_chunks(d.max_ctx, (int)hkv, G),
                                    hb * max_attn_chunks(d.max_ctx, (int)hb, G));
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  a.w = take(im.total * 2);
  a.w2 = bp ? take(image_layout(prefill_desc(d)).total * 2) : 0;
  // mixture of experts: expert codes, their row scales, the routing record
  a.w8 = moe(d) ? take(im.e8_total) : 0;
  a.esc = moe(d) ? take(im.sc_total * (mxfp4(d) ? 1 : 4)) : 0;
  a.routes = moe(d) ? take((size_t)d.max_ctx * d.n_layers * d.top_k * 4) : 0;
  a.gains = take(((size_t)d.n_layers * 2 + 1) * D * 4);
  a.rope = take((size_t)d.max_ctx * (d.head_dim / 2) * 2 * 4);
  a.kv = take((size_t)d.n_layers * 2 * hkv * d.max_ctx * d.head_dim * 2);
  // matrix prefill workspace (outside the scratch part: it lives in the
  // caller's arena for a no-allocation handle)
  if (matrix_prefill(d)) {
    const size_t mc = mp_chunk(d), F = d.d_ffn;
    a.mp_x = take(mc * D * 4);
    a.mp_h = take(mc * std::max(D, q) * 2);    // normed rows, then the attention output
    a.mp_q16 = take(mc * q * 2);
    a.mp_a = take(mc * F * 2);                   // SwiGLU output (written while the gate/up product reads mp_h)
    a.mp_s = take(mc * 4);
    a.mp_part = take(mp_part_floats(d) * 4);
  } else {
    a.mp_x = a.mp_h = a.mp_q16 = a.mp_a = a.mp_s = a.mp_part = 0;
  }
  a.x = take(B * D * 4);
  a.xg16 = take((size_t)kMaxBatch * D * 2);   // blocks of 8 rows x kMaxBatch sequences
  a.ssp = take((size_t)G * kMaxBatch * 4);
  a.qkv = take(B * 3 * q * 4);
  a.att_o = take(B * q * 4);
  a.part = take(part_rows * d.head_dim * 4);
  a.pml = take(part_rows * 2 * 4);
  // the MLP's hidden vector: d_ffn, or top_k experts' d_ffn each (batched:
  // fp16 in blocks of 8 rows x kMaxBatch sequences, whatever the batch)
  a.act = take(std::max(B * d.d_ffn * (moe(d) ? d.top_k : 1) * 4, (size_t)kMaxBatch * d.d_ffn * 2));
  if (moe(d)) a.rpart = take((size_t)G * kMoeMaxExperts * 4);
  a.logits = take(B * d.lm_vocab * 4);
  // argmax partials: [G] at batch 1, [G][kMaxBatch] for the batched kernel
  const size_t Bk = B > 1 ? (size_t)kMaxBatch : 1;
  a.amax_v = take(Bk * G * 4);
  a.amax_i = take(Bk * G * 4);
  a.tok_cur = take(B * 4);
  a.tok_out = take((size_t)d.max_ctx * B * 4);
  a.prompt = take((size_t)d.max_ctx * B * 4);
  a.ctl = take(kCtlWords * 4);
  a.srv_slot = take((size_t)kSrvSlotWords * 4);
  a.params = take(sizeof(Params));
  a.params2 = take(sizeof(Params));
  a.trace = take((size_t)G * kTraceStride * 8);
  a.total = o;
  return a;
}

}  // namespace

struct dec_handle {
  dec_model_desc desc;
  std::string err;
  int device = 0;
  int grid = 0;
  hipStream_t stream = nullptr;
  bool own_stream = false;
  void* base = nullptr;
  bool own_arena = false;
  // device address of the arena's scratch part (offsets from ar.x on): inside
  // the arena, or the fixed no-allocation array (dec_init_noalloc)
  char* scr = nullptr;
  bool noalloc = false;    // holds this device's fixed scratch array
  Arena ar;
  Image im;
  Params P;               // host copy
  Params* dP = nullptr;   // device copy read by the kernel
  Params* dP2 = nullptr;  // device copy for the batched prefill (DEC_FLAG_BATCHED_PREFILL)
  uint32_t debug = 0;
  uint32_t bar_done = 0;   // barriers completed by resident launches (wrapping)
  int pos = 0;
  bool broken = false;     // a launch failed; only dec_reset/dec_free are allowed
  bool has_prev_tok = false;
  double wall_hz = 1e8;
  // decode server (serve_idle_us > 0)
  uint32_t srv_idle_ticks = 0;  // 0: off
  Mailbox* mail = nullptr;      // host-pinned mailbox (host address)
  float* lg_host = nullptr;     // host-pinned logits [batch * lm_vocab]
  bool srv_on = false;          // a server launch is enqueued and has not been waited for
  uint32_t srv_epoch = 0;       // launches so far (tags their request slots)
  uint32_t srv_posted = 0;      // requests posted to the current launch
};

namespace {

// Which devices' fixed scratch arrays a live no-allocation handle holds.
std::atomic<bool> g_scratch_held[kMaxDevices];

int hip_fail(dec_handle* h, std::string* err, hipError_t e, const char* what) {
  if (h) h->broken = true;
  return fail(err, DEC_ERR_DEVICE, "%s failed: %s", what, hipGetErrorString(e));
}
#define HIPCHK(h, err, call) do { hipError_t e_ = (call); if (e_ != hipSuccess) return hip_fail(h, err, e_, #call); } while (0)

int launch(dec_handle* h, int pos0, int n_tok, int tok_src, int lm_last_only, int write_logits,
           const int32_t* force = nullptr) {
  Launch A;
  std::memset(&A, 0, sizeof A);
  // forced input tokens travel in the launch arguments, which are copied when
  // the kernel is enqueued: the caller's array is not read after this call
  if (force) {
    A.n_force = 1;
    for (int b = 0; b < h->desc.batch; ++b) A.force[b] = force[b];
  }
  A.pos0 = pos0;
  A.n_tok = n_tok;
  A.tok_src = tok_src;
  A.lm_last_only = lm_last_only;
  A.write_logits = write_logits;
  A.fenced = (h->debug & DEC_DEBUG_FENCED) ? 1 : 0;
  A.phase_begin = 0;
  A.phase_end = 0x7fffffff;
  A.pos_end = 0x7fffffff;
  if (h->debug & DEC_DEBUG_MULTILAUNCH) {
    // one ordinary launch per phase: the kernel boundary is the barrier
    const int ppt = phases_per_token(h->desc.n_layers);
    A.bar_base = h->bar_done;
    for (int i = 0; i < n_tok; ++i) {
      const bool lm = !lm_last_only || i == n_tok - 1;
      const int nph = kPhasesPerLayer * h->desc.n_layers + (lm ? 2 : 0);
      for (int k = 0; k < nph; ++k) {
        A.phase_begin = i * ppt + k;
        A.phase_end = A.phase_begin + 1;
        HIPCHK(h, &h->err, (hipError_t)kernel_launch_plain(h->dP, A, h->grid, kernel_kind(h->desc), h->desc.head_dim, h->stream));
      }
    }
    return DEC_OK;
  }
  A.bar_base = h->bar_done;
  HIPCHK(h, &h->err, (hipError_t)kernel_launch_resident(h->dP, A, h->grid, kernel_kind(h->desc), h->desc.head_dim, h->stream));
  h->bar_done += launch_barriers(h->desc.n_layers, n_tok, lm_last_only);
  return DEC_OK;
}

// The batched prefill: n prompt positions, kMaxBatch per token step of the
// batched kernel, the LM head and argmax for the last step only.
int launch_prefill(dec_handle* h, int n, int write_logits) {
  const int pos0 = 0, n_tok = (n + kMaxBatch - 1) / kMaxBatch, tok_src = TOK_PROMPT, lm_last_only = 1;
  Launch A;
  std::memset(&A, 0, sizeof A);
  A.pos0 = pos0;
  A.n_tok = n_tok;
  A.tok_src = tok_src;
  A.lm_last_only = lm_last_only;
  A.write_logits = write_logits;
  A.fenced = (h->debug & DEC_DEBUG_FENCED) ? 1 : 0;
  A.phase_begin = 0;
  A.phase_end = 0x7fffffff;
  A.pos_end = n;
  if (h->debug & DEC_DEBUG_MULTILAUNCH) {
    // one ordinary launch per phase: the kernel boundary is the barrier
    const int ppt = phases_per_token(h->desc.n_layers);
    A.bar_base = h->bar_done;
    for (int i = 0; i < n_tok; ++i) {
      const bool lm = !lm_last_only || i == n_tok - 1;
      const int nph = kPhasesPerLayer * h->desc.n_layers + (lm ? 2 : 0);
      for (int k = 0; k < nph; ++k) {
        A.phase_begin = i * ppt + k;
        A.phase_end = A.phase_begin + 1;
        HIPCHK(h, &h->err, (hipError_t)kernel_launch_plain(h->dP2, A, h->grid, kMaxBatch, h->desc.head_dim, h->stream));
      }
    }
    return DEC_OK;
  }
  A.bar_base = h->bar_done;
  HIPCHK(h, &h->err, (hipError_t)kernel_launch_resident(h->dP2, A, h->grid, kMaxBatch, h->desc.head_dim, h->stream));
  h->bar_done += launch_barriers(h->desc.n_layers, n_tok, lm_last_only);
  return DEC_OK;
}

// The matrix prefill of n prompt positions (already in P.prompt): chunks of
// up to kMpChunk positions, each through every layer as matrix products
// (dec_matrix.hip), then the LM-head row and greedy token of position n-1.
int launch_matrix_prefill(dec_handle* h, int n) {
  const dec_model_desc& d = h->desc;
  const Params& P = h->P;
  const int D = d.d_model, H = d.n_heads, hd = d.head_dim, q = H * hd, F = d.d_ffn, V = d.lm_vocab;
  const size_t head_elems = (size_t)d.max_ctx * hd;
  char* b = static_cast<char*>(h->base);
  float* x = reinterpret_cast<float*>(b + h->ar.mp_x);
  uint16_t* hb = reinterpret_cast<uint16_t*>(b + h->ar.mp_h);
  uint16_t* q16 = reinterpret_cast<uint16_t*>(b + h->ar.mp_q16);
  uint16_t* ab = reinterpret_cast<uint16_t*>(b + h->ar.mp_a);
  float* sb = reinterpret_cast<float*>(b + h->ar.mp_s);
  float* part = reinterpret_cast<float*>(b + h->ar.mp_part);
  const size_t part_floats = mp_part_floats(d);
  void* st = h->stream;
  auto gemm = [&](const uint16_t* A, int lda, const uint16_t* W, int M, int N, int K, const MpEpi& e) {
    MpGemm g;
    g.A = A; g.lda = lda; g.B = W; g.ldb = K;
    g.M = M; g.N = N; g.K = K; g.epi = e; g.part = part;
    mp_plan(M, N, K, part_floats, &g.shape, &g.S, &g.kc);
    return (hipError_t)mp_launch_gemm(g, st);
  };
  auto epi = [&](int mode, float* C, int ldc, const float* s) {
    MpEpi e;
    std::memset(&e, 0, sizeof e);
    e.mode = mode; e.C = C; e.ldc = ldc; e.s = s;
    return e;
  };
  const int mc = mp_chunk(d);
  int m = 0;
  for (int c0 = 0; c0 < n; c0 += mc) {
    m = std::min(mc, n - c0);
    HIPCHK(h, &h->err, (hipError_t)mp_launch_embed(P.w + P.off_E, P.prompt + c0, m, D, x, st));
    for (int l = 0; l < d.n_layers; ++l) {
      const uint16_t* W = P.w + (size_t)l * P.layer_stride;
      const float* g_attn = P.gains + (size_t)l * 2 * D;
      const float* g_ffn = g_attn + D;
      uint16_t* kc = P.kv + (size_t)l * 2 * H * head_elems;
      uint16_t* vc = kc + (size_t)H * head_elems;
      // QKV product; its epilogue rotates q and k, appends k and v to the cache, writes fp16 q
      MpEpi rope = epi(MP_EP_ROPE, nullptr, 0, sb);
      rope.H = q16; rope.ldh = q; rope.rope = P.rope; rope.kc = kc; rope.vc = vc; rope.head_elems = head_elems;
      rope.pos0 = c0; rope.q = q; rope.hd = hd;
      HIPCHK(h, &h->err, (hipError_t)mp_launch_norm(x, g_attn, m, D, d.rms_eps, hb, sb, st));
      HIPCHK(h, &h->err, gemm(hb, D, W + P.off_qkv, m, 3 * q, D, rope));
      HIPCHK(h, &h->err, (hipError_t)mp_launch_attention(q16, q, m, c0, H, hd, kc, vc, head_elems, hb, st));
      HIPCHK(h, &h->err, gemm(hb, q, W + P.off_o, m, D, q, epi(MP_EP_ACCUM, x, D, nullptr)));
      // gate/up product; its epilogue writes the fp16 SwiGLU output
      MpEpi swiglu = epi(MP_EP_SWIGLU, nullptr, 0, sb);
      swiglu.H = ab; swiglu.ldh = F;
      HIPCHK(h, &h->err, (hipError_t)mp_launch_norm(x, g_ffn, m, D, d.rms_eps, hb, sb, st));
      HIPCHK(h, &h->err, gemm(hb, D, W + P.off_gu, m, 2 * F, D, swiglu));
      HIPCHK(h, &h->err, gemm(ab, F, W + P.off_d, m, D, F, epi(MP_EP_ACCUM, x, D, nullptr)));
    }
  }
  // the last position's final norm, LM-head row and greedy token
  const float* g_final = P.gains + (size_t)d.n_layers * 2 * D;
  HIPCHK(h, &h->err, (hipError_t)mp_launch_norm(x + (size_t)(m - 1) * D, g_final, 1, D, d.rms_eps, hb, sb, st));
  HIPCHK(h, &h->err, gemm(hb, D, P.w + P.off_lm, 1, V, D, epi(MP_EP_SCALE, P.logits, V, sb)));
  HIPCHK(h, &h->err, (hipError_t)mp_launch_argmax(P.logits, V, P.tok_out + (n - 1), P.tok_cur, st));
  return DEC_OK;
}

// ---------------------------------------------------------------------------
// decode server: host side of the mailbox protocol
// ---------------------------------------------------------------------------
uint32_t mail_load(const uint32_t* p) { return __atomic_load_n(p, __ATOMIC_ACQUIRE); }

// Starts a server launch at the current position.  The previous one has been
// waited for, so no kernel reads the mailbox while it is reset.
int srv_start(dec_handle* h) {
  Mailbox* m = h->mail;
  __atomic_store_n(&m->done, 0u, __ATOMIC_RELAXED);
  __atomic_store_n(&m->ctl, 0u, __ATOMIC_SEQ_CST);
  Launch A;
  std::memset(&A, 0, sizeof A);
  A.pos0 = h->pos;
  A.n_tok = h->desc.max_ctx - h->pos;
  A.tok_src = TOK_DEVICE;
  A.fenced = (h->debug & DEC_DEBUG_FENCED) ? 1 : 0;
  A.phase_begin = 0;
  A.phase_end = 0x7fffffff;
  A.pos_end = 0x7fffffff;
  A.server = 1;
  A.srv_epoch = ++h->srv_epoch;
  if (A.srv_epoch == 0) A.srv_epoch = h->srv_epoch = 1;   // 0 would match the zeroed slots
  A.idle_ticks = h->srv_idle_ticks;
  A.bar_base = h->bar_done;
  HIPCHK(h, &h->err, (hipError_t)kernel_launch_resident(h->dP, A, h->grid, kernel_kind(h->desc), h->desc.head_dim, h->stream));
  h->srv_on = true;
  h->srv_posted = 0;
  return DEC_OK;
}

int check_device_error(dec_handle* h);

// Ends the server launch, if one runs: closes the mailbox, waits for the
// launch and adds the barriers its served requests executed.
int srv_stop(dec_handle* h) {
  if (!h->srv_on) return DEC_OK;
  __atomic_fetch_or(&h->mail->ctl, kMailClosed, __ATOMIC_SEQ_CST);
  h->srv_on = false;
  const hipError_t e = hipStreamSynchronize(h->stream);
  const uint32_t n = mail_load(&h->mail->done);
  if (n > 0) h->bar_done += launch_barriers(h->desc.n_layers, (int)n, 0);
  if (e != hipSuccess) return hip_fail(h, &h->err, e, "hipStreamSynchronize(server)");
  int rc = check_device_error(h);
  if (rc) return rc;
  if (n != h->srv_posted) {
    h->broken = true;
    return fail(&h->err, DEC_ERR_DEVICE, "server launch ended after %u of %u requests; call dec_reset", n,
                h->srv_posted);
  }
  return DEC_OK;
}

// Waits until the server launch has completed `n` requests.  The launch ends
// by itself at the latest after the idle and watchdog bounds, so the stream
// is checked now and then: a launch that ended short of n reports why.
int srv_wait(dec_handle* h, uint32_t n) {
  for (uint32_t spin = 0;; ++spin) {
    if ((int)(mail_load(&h->mail->done) - n) >= 0) return DEC_OK;
    if ((spin & 255u) == 255u) {
      const hipError_t q = hipStreamQuery(h->stream);
      if (q != hipErrorNotReady) {
        if ((int)(mail_load(&h->mail->done) - n) >= 0) return DEC_OK;
        const int rc = srv_stop(h);
        if (rc) return rc;
        h->broken = true;
        return fail(&h->err, DEC_ERR_DEVICE, "server launch ended before request %u completed; call dec_reset", n);
      }
    }
    __builtin_ia32_pause();
  }
}

// Posts one step; starts a server launch when none runs or the running one
// has closed its mailbox for idleness.
int srv_post(dec_handle* h, int flags, const int32_t* force) {
  for (int attempt = 0; attempt < 2; ++attempt) {
    if (!h->srv_on) {
      int rc = srv_start(h);
      if (rc) return rc;
    }
    Mailbox* m = h->mail;
    const uint32_t k = h->srv_posted;
    if (k >= (uint32_t)kMailRing) {
      // slot k % kMailRing last held request k - kMailRing, which must be complete
      int rc = srv_wait(h, k - kMailRing + 1);
      if (rc) return rc;
    }
    int32_t* r = m->req[k % kMailRing];
    r[0] = flags;
    for (int b = 0; b < h->desc.batch; ++b) r[1 + b] = force ? force[b] : 0;
    uint32_t expected = k;
    if (__atomic_compare_exchange_n(&m->ctl, &expected, k + 1, false, __ATOMIC_SEQ_CST, __ATOMIC_SEQ_CST)) {
      h->srv_posted = k + 1;
      return DEC_OK;
    }
    // the launch closed its mailbox at k (idle): wait for it and start another
    int rc = srv_stop(h);
    if (rc) return rc;
  }
  return fail(&h->err, DEC_ERR_DEVICE, "a fresh server launch refused a request");
}

int check_device_error(dec_handle* h) {
  uint32_t e = 0;
  HIPCHK(h, &h->err, hipMemcpyAsync(&e, h->P.ctl + kCtlErr, 4, hipMemcpyDeviceToHost, h->stream));
  HIPCHK(h, &h->err, hipStreamSynchronize(h->stream));
  if (e != 0) {
    h->broken = true;
    if ((int)e == kDevErrTimeout)
      return fail(&h->err, DEC_ERR_TIMEOUT, "a grid barrier wait passed the watchdog bound; call dec_reset");
    return fail(&h->err, DEC_ERR_DEVICE, "device raised error %d; call dec_reset", (int)e);
  }
  return DEC_OK;
}

int finish(dec_handle* h, int32_t* out_tok, int n_tok_out, float* out_logits) {
  int rc = check_device_error(h);
  if (rc) return rc;
  const size_t B = h->desc.batch;
  if (out_tok) HIPCHK(h, &h->err, hipMemcpy(out_tok, h->P.tok_out, (size_t)n_tok_out * B * 4, hipMemcpyDeviceToHost));
  if (out_logits)
    HIPCHK(h, &h->err, hipMemcpy(out_logits, h->P.logits, B * h->desc.lm_vocab * 4, hipMemcpyDeviceToHost));
  return DEC_OK;
}

int upload_weights(dec_handle* h, const dec_weights_src* src) {
  const dec_model_desc& d = h->desc;
  const int nt = n_tensors_for(d);
  std::vector<float> gains(((size_t)d.n_layers * 2 + 1) * d.d_model, 0.f);
  // Pack one layer (or the embedding / LM head) at a time into a host
  // staging image and copy it to its place in the device image.
  const size_t chunk_elems = std::max(h->im.layer_stride, (size_t)1);
  std::vector<uint16_t> stage;
  uint16_t* dev_w = reinterpret_cast<uint16_t*>(static_cast<char*>(h->base) + h->ar.w);
  std::vector<FileEntry> entries;
  FILE* f = nullptr;
  if (src->path) {
    f = std::fopen(src->path, "rb");
    if (!f) return fail(&h->err, DEC_ERR_WEIGHTS, "cannot open weight file '%s'", src->path);
    dec_model_desc fd;
    int rc = read_file_header(f, &fd, &entries, &h->err);
    if (rc) { std::fclose(f); return rc; }
    if (!same_shape(fd, d)) {
      std::fclose(f);
      return fail(&h->err, DEC_ERR_WEIGHTS, "weight file shapes differ from the model description");
    }
  }
  std::vector<uint16_t> rowbuf;
  auto fetch = [&](int idx, std::vector<uint16_t>& tmp) -> const uint16_t* {
    size_t R, C;
    tensor_shape(d, idx, &R, &C);
    if (!f) return src->host_tensors[idx];
    tmp.resize(R * C);
    if (fseeko(f, (off_t)entries[idx].offset, SEEK_SET) != 0 || std::fread(tmp.data(), 2, R * C, f) != R * C) return nullptr;
    return tmp.data();
  };
  int rc = DEC_OK;
  const Image local = h->im;
  // layers: a one-layer description has the same per-layer offsets and stride
  dec_model_desc one = d;
  one.n_layers = 1;
  const Image im1 = image_layout(one);
  // the batched prefill's tiled copy of every matrix
  const bool bp = batched_prefill(d);
  const Image im2 = image_layout(prefill_desc(d));
  dec_model_desc one2 = prefill_desc(d);
  one2.n_layers = 1;
  const Image im12 = image_layout(one2);
  uint16_t* dev_w2 = reinterpret_cast<uint16_t*>(static_cast<char*>(h->base) + h->ar.w2);
  std::vector<uint16_t> stage2;
  std::vector<float> g1(3 * (size_t)d.d_model);
  // mixture of experts: one layer's expert codes and scales
  std::vector<uint8_t> stage8(im1.e8_stride);
  std::vector<float> stagesc(im1.sc_stride);   // (MXFP4: sc_stride bytes in the first quarter)
  const size_t sc_bytes = mxfp4(d) ? local.sc_stride : local.sc_stride * 4;
  char* dev_w8 = static_cast<char*>(h->base) + h->ar.w8;
  char* dev_sc = static_cast<char*>(h->base) + h->ar.esc;
  const int per = per_layer(d);
  for (int l = 0; l < d.n_layers && rc == DEC_OK; ++l) {
    stage.assign(chunk_elems, 0);
    if (bp) stage2.assign(im12.layer_stride, 0);
    for (int kind = 0; kind < per; ++kind) {
      const int idx = 1 + per * l + kind;
      const uint16_t* t = fetch(idx, rowbuf);
      if (!t) { rc = fail(&h->err, DEC_ERR_WEIGHTS, "cannot read tensor %d from the weight file", idx); break; }
      size_t R, C;
      tensor_shape(d, idx, &R, &C);
      place_tensor(one, im1, 1 + kind, t, 0, R, stage.data(), g1.data(), stage8.data(), stagesc.data());
      if (bp) place_tensor(one2, im12, 1 + kind, t, 0, R, stage2.data(), g1.data());
    }
    if (rc != DEC_OK) break;
    std::memcpy(gains.data() + (size_t)l * 2 * d.d_model, g1.data(), 2 * (size_t)d.d_model * 4);
    hipError_t e = hipMemcpy(dev_w + (size_t)l * local.layer_stride, stage.data(), local.layer_stride * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess && bp)
      e = hipMemcpy(dev_w2 + (size_t)l * im2.layer_stride, stage2.data(), im2.layer_stride * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess && moe(d)) {
      e = hipMemcpy(dev_w8 + (size_t)l * local.e8_stride, stage8.data(), local.e8_stride, hipMemcpyHostToDevice);
      if (e == hipSuccess)
        e = hipMemcpy(dev_sc + (size_t)l * sc_bytes, stagesc.data(), sc_bytes, hipMemcpyHostToDevice);
    }
    if (e != hipSuccess) rc = hip_fail(h, &h->err, e, "hipMemcpy(weights)");
  }
  // embedding, final gain, LM head: row-major ones are copied as they are
  const int last = nt - 1;
  for (int idx : {0, last - 1, last}) {
    if (rc != DEC_OK) break;
    const uint16_t* t = fetch(idx, rowbuf);
    if (!t) { rc = fail(&h->err, DEC_ERR_WEIGHTS, "cannot read tensor %d from the weight file", idx); break; }
    size_t R, C;
    tensor_shape(d, idx, &R, &C);
    if (idx == last - 1) {
      place_tensor(d, local, idx, t, 0, R, nullptr, gains.data());
      continue;
    }
    const size_t off = idx == 0 ? local.off_E : local.off_lm;
    hipError_t e;
    if (idx == last && local.tiled) {
      // tiles: pack into a staging copy of the LM head's region first
      stage.assign(local.total - local.off_lm, 0);
      for (size_t r = 0; r < R; ++r) put_row(stage.data(), 0, r, t + r * C, C, true);
      e = hipMemcpy(dev_w + off, stage.data(), stage.size() * 2, hipMemcpyHostToDevice);
    } else {
      e = hipMemcpy(dev_w + off, t, R * C * 2, hipMemcpyHostToDevice);
    }
    if (e == hipSuccess && bp) {
      // the tiled copy: the embedding as it is, the LM head in tiles
      if (idx == 0) {
        e = hipMemcpy(dev_w2 + im2.off_E, t, R * C * 2, hipMemcpyHostToDevice);
      } else {
        stage.assign(im2.total - im2.off_lm, 0);
        for (size_t r = 0; r < R; ++r) put_row(stage.data(), 0, r, t + r * C, C, true);
        e = hipMemcpy(dev_w2 + im2.off_lm, stage.data(), stage.size() * 2, hipMemcpyHostToDevice);
      }
    }
    if (e != hipSuccess) rc = hip_fail(h, &h->err, e, "hipMemcpy(embedding/LM head)");
  }
  if (f) std::fclose(f);
  if (rc) return rc;
  HIPCHK(h, &h->err, hipMemcpy(static_cast<char*>(h->base) + h->ar.gains, gains.data(), gains.size() * 4, hipMemcpyHostToDevice));
  return DEC_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int32_t dec_abi_version(void) { return DEC_ABI_VERSION; }

int dec_check_desc(const dec_model_desc* desc) { return check_desc_impl(desc, nullptr); }

int dec_arena_bytes(const dec_model_desc* desc, int32_t grid, size_t* out_bytes) {
  if (!out_bytes) return fail(nullptr, DEC_ERR_INVALID_ARG, "out_bytes is NULL");
  int rc = check_desc_impl(desc, nullptr);
  if (rc) return rc;
  if (grid < 0 || grid > 1024) return fail(nullptr, DEC_ERR_INVALID_ARG, "grid must be in [0, 1024]");
  *out_bytes = arena_layout(*desc, grid ? grid : 256).total;
  return DEC_OK;
}

int dec_packed_bytes(const dec_model_desc* desc, size_t* out_bytes) {
  if (!out_bytes) return fail(nullptr, DEC_ERR_INVALID_ARG, "out_bytes is NULL");
  int rc = check_desc_impl(desc, nullptr);
  if (rc) return rc;
  if (moe(*desc)) return fail(nullptr, DEC_ERR_UNSUPPORTED, "the packed fp16 image is for dense models");
  *out_bytes = image_layout(*desc).total * 2;
  return DEC_OK;
}

int dec_pack(const dec_model_desc* desc, const uint16_t* const* host_tensors, int32_t n_tensors, void* dst, size_t dst_bytes) {
  int rc = check_desc_impl(desc, nullptr);
  if (rc) return rc;
  if (moe(*desc)) return fail(nullptr, DEC_ERR_UNSUPPORTED, "the packed fp16 image is for dense models");
  if (!host_tensors || !dst) return fail(nullptr, DEC_ERR_INVALID_ARG, "NULL tensor list or destination");
  if (n_tensors != n_tensors_for(*desc))
    return fail(nullptr, DEC_ERR_WEIGHTS, "expected %d tensors, got %d", n_tensors_for(*desc), n_tensors);
  const Image im = image_layout(*desc);
  if (dst_bytes < im.total * 2) return fail(nullptr, DEC_ERR_INVALID_ARG, "destination smaller than %zu bytes", im.total * 2);
  std::memset(dst, 0, im.total * 2);
  std::vector<float> gains(((size_t)desc->n_layers * 2 + 1) * desc->d_model);
  for (int i = 0; i < n_tensors; ++i) {
    if (!host_tensors[i]) return fail(nullptr, DEC_ERR_WEIGHTS, "tensor %d is NULL", i);
    size_t R, C;
    tensor_shape(*desc, i, &R, &C);
    place_tensor(*desc, im, i, host_tensors[i], 0, R, static_cast<uint16_t*>(dst), gains.data());
  }
  return DEC_OK;
}

int dec_weights_file_check(const char* path, dec_model_desc* out_desc) {
  if (!path || !out_desc) return fail(nullptr, DEC_ERR_INVALID_ARG, "NULL path or output");
  FILE* f = std::fopen(path, "rb");
  if (!f) return fail(nullptr, DEC_ERR_WEIGHTS, "cannot open weight file '%s'", path);
  std::vector<FileEntry> entries;
  int rc = read_file_header(f, out_desc, &entries, nullptr);
  std::fclose(f);
  return rc;
}

}  // extern "C"
#pragma GCC visibility pop

namespace {

// dec_init and dec_init_noalloc.  noalloc: the caller's arena holds the
// weights, gains, rotary table and KV cache (the arena's leading part, up to
// ar.x); the rest of the layout (ar.x .. ) lives in this device's fixed
// scratch array instead, and no device memory is allocated.
int init_impl(const dec_model_desc* desc, const dec_weights_src* weights, const dec_init_opts* opts, dec_handle** out,
              bool noalloc) {
  if (!out) return fail(nullptr, DEC_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int rc = check_desc_impl(desc, nullptr);
  if (rc) return rc;
  if (!weights) return fail(nullptr, DEC_ERR_INVALID_ARG, "weights is NULL");
  if ((weights->path == nullptr) == (weights->host_tensors == nullptr))
    return fail(nullptr, DEC_ERR_INVALID_ARG, "exactly one of weights->path and weights->host_tensors must be set");
  if (moe(*desc) && weights->path)
    return fail(nullptr, DEC_ERR_UNSUPPORTED, "a mixture-of-experts model comes from host tensors, not a DECW file");
  if (moe(*desc) && noalloc)
    return fail(nullptr, DEC_ERR_UNSUPPORTED, "a mixture-of-experts model is not served by dec_init_noalloc");
  if (weights->host_tensors) {
    if (weights->n_tensors != n_tensors_for(*desc))
      return fail(nullptr, DEC_ERR_WEIGHTS, "expected %d tensors, got %d", n_tensors_for(*desc), weights->n_tensors);
    for (int i = 0; i < weights->n_tensors; ++i)
      if (!weights->host_tensors[i]) return fail(nullptr, DEC_ERR_WEIGHTS, "tensor %d is NULL", i);
  } else {
    FILE* f = std::fopen(weights->path, "rb");
    if (!f) return fail(nullptr, DEC_ERR_WEIGHTS, "cannot open weight file '%s'", weights->path);
    dec_model_desc fd;
    std::vector<FileEntry> entries;
    rc = read_file_header(f, &fd, &entries, nullptr);
    std::fclose(f);
    if (rc) return rc;
    if (!same_shape(fd, *desc)) return fail(nullptr, DEC_ERR_WEIGHTS, "weight file shapes differ from the model description");
  }
  dec_init_opts o;
  std::memset(&o, 0, sizeof o);
  if (opts) o = *opts;
  if (o.grid < 0 || o.grid > 1024) return fail(nullptr, DEC_ERR_INVALID_ARG, "grid must be in [0, 1024]");
  if (o.watchdog_us < 0) return fail(nullptr, DEC_ERR_INVALID_ARG, "watchdog_us must be >= 0");
  if (o.debug_flags & ~(DEC_DEBUG_MULTILAUNCH | DEC_DEBUG_TRACE | DEC_DEBUG_FENCED | DEC_DEBUG_STRESS))
    return fail(nullptr, DEC_ERR_INVALID_ARG, "unknown debug flags 0x%x", o.debug_flags);
  if (moe(*desc) && (o.debug_flags & DEC_DEBUG_MULTILAUNCH))
    return fail(nullptr, DEC_ERR_UNSUPPORTED, "a mixture-of-experts model keeps its routing on chip between phases: "
                "not with DEC_DEBUG_MULTILAUNCH");
  if ((o.debug_flags & DEC_DEBUG_STRESS) && (o.debug_flags & DEC_DEBUG_MULTILAUNCH))
    return fail(nullptr, DEC_ERR_INVALID_ARG, "DEC_DEBUG_STRESS needs the resident kernel (not DEC_DEBUG_MULTILAUNCH)");
  if (o.serve_idle_us < 0 || o.serve_idle_us > 10000000)
    return fail(nullptr, DEC_ERR_INVALID_ARG, "serve_idle_us must be in [0, 10000000]");
  if (o.serve_idle_us > 0 && noalloc)
    return fail(nullptr, DEC_ERR_INVALID_ARG, "the decode server allocates host-pinned memory: not with dec_init_noalloc");
  if (o.serve_idle_us > 0 && (o.debug_flags & DEC_DEBUG_MULTILAUNCH))
    return fail(nullptr, DEC_ERR_INVALID_ARG, "the decode server is one resident launch: not with DEC_DEBUG_MULTILAUNCH");
  if (noalloc && (!o.arena || !o.stream))
    return fail(nullptr, DEC_ERR_INVALID_ARG, "dec_init_noalloc needs a caller arena and a caller stream");
  if (noalloc && (o.device < 0 || o.device >= kMaxDevices))
    return fail(nullptr, DEC_ERR_NO_DEVICE, "device %d is past the %d devices the fixed scratch serves", o.device,
                kMaxDevices);

  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return fail(nullptr, DEC_ERR_NO_DEVICE, "no HIP device visible");
  if (o.device < 0 || o.device >= ndev) return fail(nullptr, DEC_ERR_NO_DEVICE, "device %d not present (%d visible)", o.device, ndev);
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, o.device) != hipSuccess) return fail(nullptr, DEC_ERR_NO_DEVICE, "cannot query device %d", o.device);
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(nullptr, DEC_ERR_NO_DEVICE, "device %d is %s; this library is built for gfx950", o.device, prop.gcnArchName);
  if (hipSetDevice(o.device) != hipSuccess) return fail(nullptr, DEC_ERR_NO_DEVICE, "hipSetDevice(%d) failed", o.device);

  dec_handle* h = new (std::nothrow) dec_handle();
  if (!h) return fail(nullptr, DEC_ERR_OOM, "host allocation failed");
  h->desc = *desc;
  h->device = o.device;
  h->debug = o.debug_flags;
  const int cus = prop.multiProcessorCount;
  h->grid = o.grid ? o.grid : cus;
  auto bail = [&](int code) {
    g_err = h->err;
    dec_free(h);
    return code;
  };
  // the resident kernel needs every workgroup co-resident
  int coop = 0;
  (void)hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, o.device);
  if (!coop && !(h->debug & DEC_DEBUG_MULTILAUNCH)) {
    fail(&h->err, DEC_ERR_UNSUPPORTED, "device lacks cooperative launch");
    return bail(DEC_ERR_UNSUPPORTED);
  }
  hipError_t e = (hipError_t)kernel_prepare();
  if (e == hipSuccess && matrix_prefill(*desc)) e = (hipError_t)mp_prepare();
  if (e != hipSuccess) { hip_fail(h, &h->err, e, "hipFuncSetAttribute"); return bail(DEC_ERR_DEVICE); }
  int per_cu = 0;
  e = (hipError_t)kernel_blocks_per_cu(kernel_kind(*desc), desc->head_dim, &per_cu);
  if (e != hipSuccess) { hip_fail(h, &h->err, e, "hipOccupancyMaxActiveBlocksPerMultiprocessor"); return bail(DEC_ERR_DEVICE); }
  if (per_cu < 1 || h->grid > per_cu * cus) {
    fail(&h->err, DEC_ERR_UNSUPPORTED, "grid %d exceeds co-resident capacity %d x %d", h->grid, per_cu, cus);
    return bail(DEC_ERR_UNSUPPORTED);
  }
  {
    // attention gives every (column, head) pair at least one workgroup
    const long long pairs = (long long)(batched_prefill(*desc) ? kMaxBatch : desc->batch) * desc->n_heads;
    if (pairs > h->grid) {
      fail(&h->err, DEC_ERR_UNSUPPORTED, "grid %d is smaller than the %lld (sequence or position, head) pairs",
           h->grid, pairs);
      return bail(DEC_ERR_UNSUPPORTED);
    }
  }
  {
    // per-workgroup GEMV results (every sequence) and residual rows live in
    // fixed LDS buffers; the batch kernel keeps kMaxBatch sequences' slots
    auto per_wg = [&](long long n) { return (n + h->grid - 1) / h->grid; };
    const long long q = (long long)desc->n_heads * desc->head_dim;
    const bool tiled = desc->batch > 1;
    const long long mb = tiled ? kMaxBatch : 1;
    // rows a workgroup owns in a matrix of `rows` rows: row pairs, or whole 16-row groups
    auto rows_wg = [&](long long rows) {
      return tiled ? kTileRows * per_wg((rows + kTileRows - 1) / kTileRows) : 2 * per_wg(rows / 2);
    };
    long long need_out = mb * std::max({rows_wg(3 * q), rows_wg(desc->d_model), rows_wg(2LL * desc->d_ffn),
                                        rows_wg(desc->lm_vocab)});
    if (moe(*desc)) {
      // the router's logits, then the workgroup's gate/up row pairs of its
      // expert slot (every slot has at least h->grid / top_k workgroups)
      if (h->grid < desc->top_k) {
        fail(&h->err, DEC_ERR_UNSUPPORTED, "grid %d is smaller than top_k", h->grid);
        return bail(DEC_ERR_UNSUPPORTED);
      }
      const long long wg_slot = h->grid / desc->top_k;
      need_out = std::max(need_out, (long long)kMoeOutPairs + 2 * ((desc->d_ffn + wg_slot - 1) / wg_slot));
      if ((long long)desc->n_experts * rows_wg(desc->d_model) > kMoeWrElems) {
        fail(&h->err, DEC_ERR_UNSUPPORTED, "grid %d too small for this model (a workgroup would stage %lld router "
             "weights)", h->grid, (long long)desc->n_experts * rows_wg(desc->d_model));
        return bail(DEC_ERR_UNSUPPORTED);
      }
      if ((long long)desc->top_k * rows_wg(desc->d_model) > kMoeScaleFloats) {
        fail(&h->err, DEC_ERR_UNSUPPORTED, "grid %d too small for this model (a workgroup would stage %lld down-row "
             "scales)", h->grid, (long long)desc->top_k * rows_wg(desc->d_model));
        return bail(DEC_ERR_UNSUPPORTED);
      }
    }
    long long need_own = mb * rows_wg(desc->d_model);
    if (batched_prefill(*desc)) {
      // the batched prefill runs the tiled kernel with kMaxBatch columns
      auto rows_t = [&](long long rows) { return kTileRows * per_wg((rows + kTileRows - 1) / kTileRows); };
      need_out = std::max(need_out, (long long)kMaxBatch * std::max({rows_t(3 * q), rows_t(desc->d_model),
                                                                      rows_t(2LL * desc->d_ffn), rows_t(desc->lm_vocab)}));
      need_own = std::max(need_own, (long long)kMaxBatch * rows_t(desc->d_model));
    }
    if (need_out > kOutFloats || need_own > kOwnFloats) {
      fail(&h->err, DEC_ERR_UNSUPPORTED, "grid %d too small for this model (a workgroup would own %lld outputs)",
           h->grid, need_out);
      return bail(DEC_ERR_UNSUPPORTED);
    }
  }
  if (o.stream) {
    h->stream = static_cast<hipStream_t>(o.stream);
  } else {
    e = hipStreamCreateWithFlags(&h->stream, hipStreamNonBlocking);
    if (e != hipSuccess) { hip_fail(h, &h->err, e, "hipStreamCreate"); return bail(DEC_ERR_DEVICE); }
    h->own_stream = true;
  }
  h->im = image_layout(*desc);
  h->ar = arena_layout(*desc, h->grid);
  // the scratch part: everything from the residual stream on (the trace only when asked for)
  const size_t scratch_end = (h->debug & DEC_DEBUG_TRACE) ? h->ar.total : h->ar.trace;
  const size_t scratch_bytes = scratch_end - h->ar.x;
  if (noalloc && scratch_bytes > kNoallocScratchBytes) {
    fail(&h->err, DEC_ERR_UNSUPPORTED, "this description needs %zu bytes of scratch; the fixed no-allocation array "
         "holds %zu", scratch_bytes, kNoallocScratchBytes);
    return bail(DEC_ERR_UNSUPPORTED);
  }
  const size_t need = noalloc ? h->ar.x : h->ar.total;
  if (o.arena) {
    if (reinterpret_cast<uintptr_t>(o.arena) % kAlign) { fail(&h->err, DEC_ERR_INVALID_ARG, "arena is not 256-byte aligned"); return bail(DEC_ERR_INVALID_ARG); }
    if (o.arena_bytes < need) {
      fail(&h->err, DEC_ERR_OOM, "arena of %zu bytes is smaller than the %zu needed", o.arena_bytes, need);
      return bail(DEC_ERR_OOM);
    }
    h->base = o.arena;
  } else {
    e = hipMalloc(&h->base, h->ar.total);
    if (e != hipSuccess) {
      h->base = nullptr;
      fail(&h->err, DEC_ERR_OOM, "hipMalloc of %zu bytes failed: %s", h->ar.total, hipGetErrorString(e));
      return bail(DEC_ERR_OOM);
    }
    h->own_arena = true;
  }
  char* b = static_cast<char*>(h->base);
  if (noalloc) {
    bool held = false;
    if (!g_scratch_held[o.device].compare_exchange_strong(held, true)) {
      fail(&h->err, DEC_ERR_STATE, "another no-allocation handle holds device %d's scratch array", o.device);
      return bail(DEC_ERR_STATE);
    }
    h->noalloc = true;
    void* p = nullptr;
    e = (hipError_t)kernel_scratch(o.device, &p);
    if (e != hipSuccess) { hip_fail(h, &h->err, e, "hipGetSymbolAddress(scratch)"); return bail(DEC_ERR_DEVICE); }
    h->scr = static_cast<char*>(p);
    // the array keeps its previous user's contents: clear what this handle uses
    e = hipMemsetAsync(h->scr, 0, scratch_bytes, h->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess) { hip_fail(h, &h->err, e, "hipMemsetAsync(scratch)"); return bail(DEC_ERR_DEVICE); }
  } else {
    h->scr = b + h->ar.x;
    // zero activations and control words (weights and cache are overwritten)
    e = hipMemset(h->scr, 0, h->ar.total - h->ar.x);
    if (e != hipSuccess) { hip_fail(h, &h->err, e, "hipMemset"); return bail(DEC_ERR_DEVICE); }
  }
  // device address of a scratch-part offset of the layout
  auto sc = [&](size_t off) { return h->scr + (off - h->ar.x); };
  rc = upload_weights(h, weights);
  if (rc) return bail(rc);
  // rotary table: cos/sin(p * base^(-2i/hd)) in double, stored as fp32
  {
    const int half = desc->head_dim / 2;
    std::vector<float> tab((size_t)desc->max_ctx * half * 2);
    for (int p = 0; p < desc->max_ctx; ++p)
      for (int i = 0; i < half; ++i) {
        const double theta = std::pow((double)desc->rope_base, -2.0 * i / desc->head_dim);
        const double ang = (double)p * theta;
        tab[((size_t)p * half + i) * 2] = (float)std::cos(ang);
        tab[((size_t)p * half + i) * 2 + 1] = (float)std::sin(ang);
      }
    e = hipMemcpy(b + h->ar.rope, tab.data(), tab.size() * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) { hip_fail(h, &h->err, e, "hipMemcpy(rope)"); return bail(DEC_ERR_DEVICE); }
  }
  int wall_khz = 100000;
  (void)hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, o.device);
  if (wall_khz <= 0) wall_khz = 100000;
  const double wd_us = o.watchdog_us ? (double)o.watchdog_us : 2.0e6;
  const double ticks = wd_us * wall_khz / 1000.0;
  Params& P = h->P;
  P.L = desc->n_layers; P.d = desc->d_model; P.H = desc->n_heads; P.hd = desc->head_dim; P.F = desc->d_ffn;
  P.E = desc->n_experts; P.topk = desc->top_k; P.Fe = desc->d_ffn;
  if (moe(*desc)) {
    P.F = desc->top_k * desc->d_ffn;   // the down product's input: every chosen expert's hidden vector
    P.w8 = reinterpret_cast<const uint8_t*>(b + h->ar.w8);
    P.e8_stride = h->im.e8_stride; P.e8_d = h->im.e8_d;
    P.esc = reinterpret_cast<const float*>(b + h->ar.esc);
    P.sc_stride = h->im.sc_stride; P.sc_d = h->im.sc_d;
    P.routes = reinterpret_cast<int32_t*>(b + h->ar.routes);
    P.rpart = reinterpret_cast<float*>(sc(h->ar.rpart));
    P.mx = mxfp4(*desc) ? 1 : 0;
    P.xsc = reinterpret_cast<const uint8_t*>(b + h->ar.esc);
    P.xsc_stride = h->im.sc_stride;
    P.xsc_d = h->im.sc_d;
    e = hipMemset(P.routes, 0xFF, (size_t)desc->max_ctx * desc->n_layers * desc->top_k * 4);
    if (e != hipSuccess) { hip_fail(h, &h->err, e, "hipMemset(routes)"); return bail(DEC_ERR_DEVICE); }
  }
  P.V = desc->vocab; P.Vlm = desc->lm_vocab; P.max_ctx = desc->max_ctx; P.q = desc->n_heads * desc->head_dim;
  P.eps = desc->rms_eps;
  P.w = reinterpret_cast<const uint16_t*>(b + h->ar.w);
  P.layer_stride = h->im.layer_stride;
  P.off_qkv = h->im.off_qkv; P.off_o = h->im.off_o; P.off_gu = h->im.off_gu; P.off_d = h->im.off_d;
  P.off_E = h->im.off_E; P.off_lm = h->im.off_lm;
  P.gains = reinterpret_cast<const float*>(b + h->ar.gains);
  P.rope = reinterpret_cast<const float*>(b + h->ar.rope);
  P.B = desc->batch;
  P.kv = reinterpret_cast<uint16_t*>(b + h->ar.kv);
  P.x = reinterpret_cast<float*>(sc(h->ar.x));
  P.xg16 = reinterpret_cast<uint16_t*>(sc(h->ar.xg16));
  P.ssp = reinterpret_cast<float*>(sc(h->ar.ssp));
  P.qkv = reinterpret_cast<float*>(sc(h->ar.qkv));
  P.att_o = reinterpret_cast<float*>(sc(h->ar.att_o));
  P.att_o16 = reinterpret_cast<uint16_t*>(sc(h->ar.att_o));
  P.part = reinterpret_cast<float*>(sc(h->ar.part));
  P.pml = reinterpret_cast<float*>(sc(h->ar.pml));
  P.act = reinterpret_cast<float*>(sc(h->ar.act));
  P.act16 = reinterpret_cast<uint16_t*>(sc(h->ar.act));
  P.logits = reinterpret_cast<float*>(sc(h->ar.logits));
  P.amax_v = reinterpret_cast<float*>(sc(h->ar.amax_v));
  P.amax_i = reinterpret_cast<int*>(sc(h->ar.amax_i));
  P.tok_cur = reinterpret_cast<int*>(sc(h->ar.tok_cur));
  P.tok_out = reinterpret_cast<int*>(sc(h->ar.tok_out));
  P.prompt = reinterpret_cast<const int*>(sc(h->ar.prompt));
  P.ctl = reinterpret_cast<uint32_t*>(sc(h->ar.ctl));
  P.max_chunks = max_attn_chunks(desc->max_ctx, desc->batch * desc->n_heads, h->grid);
  P.watchdog_ticks = (uint32_t)std::min(ticks, 4.0e9);
  P.trace = (h->debug & DEC_DEBUG_TRACE) ? reinterpret_cast<uint64_t*>(sc(h->ar.trace)) : nullptr;
  P.trace_stride = kTraceStride;
  h->wall_hz = (double)wall_khz * 1000.0;
  P.cols_pos = 0;
  P.stress = (h->debug & DEC_DEBUG_STRESS) ? 1 : 0;
  P.srv_slot = reinterpret_cast<int32_t*>(sc(h->ar.srv_slot));
  if (o.serve_idle_us > 0) {
    // decode server: mailbox and logits in host-pinned memory the device maps
    const unsigned fl = hipHostMallocMapped | hipHostMallocCoherent;
    void* dm = nullptr;
    void* dl = nullptr;
    e = hipHostMalloc(reinterpret_cast<void**>(&h->mail), sizeof(Mailbox), fl);
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&h->lg_host), (size_t)desc->batch * desc->lm_vocab * 4, fl);
    if (e != hipSuccess) {
      fail(&h->err, DEC_ERR_OOM, "hipHostMalloc (server mailbox) failed: %s", hipGetErrorString(e));
      return bail(DEC_ERR_OOM);
    }
    std::memset(h->mail, 0, sizeof(Mailbox));
    e = hipHostGetDevicePointer(&dm, h->mail, 0);
    if (e == hipSuccess) e = hipHostGetDevicePointer(&dl, h->lg_host, 0);
    if (e != hipSuccess) { hip_fail(h, &h->err, e, "hipHostGetDevicePointer"); return bail(DEC_ERR_DEVICE); }
    P.mail = static_cast<Mailbox*>(dm);
    P.lg_sys = static_cast<float*>(dl);
    h->srv_idle_ticks = (uint32_t)std::min((double)o.serve_idle_us * wall_khz / 1000.0, 4.0e9);
    if (h->srv_idle_ticks == 0) h->srv_idle_ticks = 1;
  }
  h->dP = reinterpret_cast<Params*>(sc(h->ar.params));
  e = hipMemcpy(h->dP, &P, sizeof(Params), hipMemcpyHostToDevice);
  if (e != hipSuccess) { hip_fail(h, &h->err, e, "hipMemcpy(params)"); return bail(DEC_ERR_DEVICE); }
  if (batched_prefill(*desc)) {
    // the batched prefill: same buffers and cache, tiled weights, kMaxBatch
    // columns that are consecutive positions of the sequence
    const Image im2 = image_layout(prefill_desc(*desc));
    Params P2 = P;
    P2.w = reinterpret_cast<const uint16_t*>(b + h->ar.w2);
    P2.layer_stride = im2.layer_stride;
    P2.off_qkv = im2.off_qkv; P2.off_o = im2.off_o; P2.off_gu = im2.off_gu; P2.off_d = im2.off_d;
    P2.off_E = im2.off_E; P2.off_lm = im2.off_lm;
    P2.B = kMaxBatch;
    P2.cols_pos = 1;
    P2.max_chunks = max_attn_chunks(desc->max_ctx, kMaxBatch * desc->n_heads, h->grid);
    h->dP2 = reinterpret_cast<Params*>(sc(h->ar.params2));
    e = hipMemcpy(h->dP2, &P2, sizeof(Params), hipMemcpyHostToDevice);
    if (e != hipSuccess) { hip_fail(h, &h->err, e, "hipMemcpy(params)"); return bail(DEC_ERR_DEVICE); }
    per_cu = 0;
    e = (hipError_t)kernel_blocks_per_cu(kMaxBatch, desc->head_dim, &per_cu);
    if (e != hipSuccess || per_cu < 1 || h->grid > per_cu * cus) {
      fail(&h->err, DEC_ERR_UNSUPPORTED, "the batched prefill kernel cannot keep %d workgroups resident", h->grid);
      return bail(DEC_ERR_UNSUPPORTED);
    }
  }
  if (hipDeviceSynchronize() != hipSuccess) { fail(&h->err, DEC_ERR_DEVICE, "device synchronize failed after upload"); return bail(DEC_ERR_DEVICE); }
  *out = h;
  return DEC_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int dec_init(const dec_model_desc* desc, const dec_weights_src* weights, const dec_init_opts* opts, dec_handle** out) {
  return init_impl(desc, weights, opts, out, false);
}

int dec_init_noalloc(const dec_model_desc* desc, const dec_weights_src* weights, const dec_init_opts* opts,
                     dec_handle** out) {
  return init_impl(desc, weights, opts, out, true);
}

int dec_prefill(dec_handle* h, const int32_t* tokens, int32_t n, int32_t* out_tok, float* out_logits) {
  if (!h) return fail(nullptr, DEC_ERR_INVALID_ARG, "handle is NULL");
  if (!tokens || !out_tok) return fail(&h->err, DEC_ERR_INVALID_ARG, "tokens and out_tok are required");
  if (h->broken) return fail(&h->err, DEC_ERR_STATE, "handle is in an error state; call dec_reset");
  if (h->pos != 0) return fail(&h->err, DEC_ERR_STATE, "prefill needs position 0 (call dec_reset)");
  if (n < 1) return fail(&h->err, DEC_ERR_INVALID_ARG, "n must be >= 1");
  if (int rc0 = srv_stop(h)) return rc0;
  if (n > h->desc.max_ctx) return fail(&h->err, DEC_ERR_CONTEXT_FULL, "prompt of %d tokens exceeds max_ctx %d", n, h->desc.max_ctx);
  const int B = h->desc.batch;
  for (long long i = 0; i < (long long)n * B; ++i)
    if (tokens[i] < 0 || tokens[i] >= h->desc.vocab)
      return fail(&h->err, DEC_ERR_TOKEN_RANGE, "prompt token %lld = %d outside [0, %d)", i, tokens[i], h->desc.vocab);
  HIPCHK(h, &h->err, hipMemcpyAsync(const_cast<int*>(h->P.prompt), tokens, (size_t)n * B * 4, hipMemcpyHostToDevice,
                                    h->stream));
  if (matrix_prefill(h->desc)) {
    int rc = launch_matrix_prefill(h, n);
    if (rc) return rc;
    h->pos = n;
    h->has_prev_tok = true;
    rc = check_device_error(h);
    if (rc) return rc;
    HIPCHK(h, &h->err, hipMemcpy(out_tok, h->P.tok_out + (n - 1), 4, hipMemcpyDeviceToHost));
    if (out_logits)
      HIPCHK(h, &h->err, hipMemcpy(out_logits, h->P.logits, (size_t)h->desc.lm_vocab * 4, hipMemcpyDeviceToHost));
    return DEC_OK;
  }
  if (h->dP2) {
    // kMaxBatch positions per step; the last step's last live column is position n-1
    int rc = launch_prefill(h, n, out_logits != nullptr);
    if (rc) return rc;
    h->pos = n;
    h->has_prev_tok = true;
    rc = check_device_error(h);
    if (rc) return rc;
    const int last = (n - 1) % kMaxBatch;
    const size_t step = (size_t)(n - 1) / kMaxBatch;
    HIPCHK(h, &h->err, hipMemcpy(out_tok, h->P.tok_out + step * kMaxBatch + last, 4, hipMemcpyDeviceToHost));
    if (out_logits)
      HIPCHK(h, &h->err, hipMemcpy(out_logits, h->P.logits + (size_t)last * h->desc.lm_vocab,
                                   (size_t)h->desc.lm_vocab * 4, hipMemcpyDeviceToHost));
    return DEC_OK;
  }
  int rc = launch(h, 0, n, TOK_PROMPT, 1, out_logits != nullptr);
  if (rc) return rc;
  h->pos = n;
  h->has_prev_tok = true;
  // the launch computed token index n-1's argmax
  rc = check_device_error(h);
  if (rc) return rc;
  HIPCHK(h, &h->err, hipMemcpy(out_tok, h->P.tok_out + (size_t)(n - 1) * B, (size_t)B * 4, hipMemcpyDeviceToHost));
  if (out_logits)
    HIPCHK(h, &h->err, hipMemcpy(out_logits, h->P.logits, (size_t)B * h->desc.lm_vocab * 4, hipMemcpyDeviceToHost));
  return DEC_OK;
}

int dec_step(dec_handle* h, const int32_t* force_tok, int32_t* out_tok, float* out_logits) {
  if (!h) return fail(nullptr, DEC_ERR_INVALID_ARG, "handle is NULL");
  if (h->broken) return fail(&h->err, DEC_ERR_STATE, "handle is in an error state; call dec_reset");
  if (h->pos >= h->desc.max_ctx) return fail(&h->err, DEC_ERR_CONTEXT_FULL, "context is full (%d positions)", h->desc.max_ctx);
  if (!force_tok && !h->has_prev_tok) return fail(&h->err, DEC_ERR_STATE, "no previous token: prefill first or pass force_tok");
  if (force_tok) {
    for (int b = 0; b < h->desc.batch; ++b)
      if (force_tok[b] < 0 || force_tok[b] >= h->desc.vocab)
        return fail(&h->err, DEC_ERR_TOKEN_RANGE, "token %d of sequence %d outside [0, %d)", force_tok[b], b,
                    h->desc.vocab);
  }
  if (h->srv_idle_ticks) {
    // decode server: post the step; wait only for what the caller asked for
    const int flags = (force_tok ? kReqForce : 0) | (out_logits ? kReqLogits : 0);
    int rc = srv_post(h, flags, force_tok);
    if (rc) return rc;
    h->pos += 1;
    h->has_prev_tok = true;
    if (!out_tok && !out_logits) return DEC_OK;
    const uint32_t k = h->srv_posted - 1;
    rc = srv_wait(h, k + 1);
    if (rc) return rc;
    const size_t B = h->desc.batch;
    if (out_tok)
      for (size_t b = 0; b < B; ++b) out_tok[b] = __atomic_load_n(&h->mail->tok[k % kMailRing][b], __ATOMIC_RELAXED);
    if (out_logits) std::memcpy(out_logits, h->lg_host, B * h->desc.lm_vocab * 4);
    return DEC_OK;
  }
  int rc = launch(h, h->pos, 1, TOK_DEVICE, 0, out_logits != nullptr, force_tok);
  if (rc) return rc;
  h->pos += 1;
  h->has_prev_tok = true;
  if (!out_tok && !out_logits) return DEC_OK;
  return finish(h, out_tok, 1, out_logits);
}

int dec_generate(dec_handle* h, int32_t n_steps, int32_t* out_toks) {
  if (!h) return fail(nullptr, DEC_ERR_INVALID_ARG, "handle is NULL");
  if (!out_toks) return fail(&h->err, DEC_ERR_INVALID_ARG, "out_toks is required");
  if (h->broken) return fail(&h->err, DEC_ERR_STATE, "handle is in an error state; call dec_reset");
  if (n_steps < 1) return fail(&h->err, DEC_ERR_INVALID_ARG, "n_steps must be >= 1");
  if (!h->has_prev_tok) return fail(&h->err, DEC_ERR_STATE, "no previous token: prefill first");
  if ((long long)h->pos + n_steps > h->desc.max_ctx)
    return fail(&h->err, DEC_ERR_CONTEXT_FULL, "%d steps from position %d pass max_ctx %d", n_steps, h->pos, h->desc.max_ctx);
  if (int rc0 = srv_stop(h)) return rc0;
  int rc = launch(h, h->pos, n_steps, TOK_DEVICE, 0, 0);
  if (rc) return rc;
  h->pos += n_steps;
  return finish(h, out_toks, n_steps, nullptr);
}

int dec_sync(dec_handle* h) {
  if (!h) return fail(nullptr, DEC_ERR_INVALID_ARG, "handle is NULL");
  if (h->broken) return fail(&h->err, DEC_ERR_STATE, "handle is in an error state; call dec_reset");
  if (h->srv_on) return srv_stop(h);
  return check_device_error(h);
}

int dec_reset(dec_handle* h) {
  if (!h) return fail(nullptr, DEC_ERR_INVALID_ARG, "handle is NULL");
  (void)srv_stop(h);   // an error it reports leaves the handle broken, which the reset clears
  hipError_t e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return fail(&h->err, DEC_ERR_DEVICE, "hipStreamSynchronize failed: %s", hipGetErrorString(e));
  if (h->broken) {
    // barrier counters may be mid-epoch after an aborted launch: restart them
    e = hipMemset(h->P.ctl, 0, kCtlWords * 4);
    if (e != hipSuccess) return fail(&h->err, DEC_ERR_DEVICE, "hipMemset(control) failed: %s", hipGetErrorString(e));
    h->bar_done = 0;
    h->broken = false;
  }
  if (moe(h->desc)) {
    e = hipMemset(h->P.routes, 0xFF, (size_t)h->desc.max_ctx * h->desc.n_layers * h->desc.top_k * 4);
    if (e != hipSuccess) return fail(&h->err, DEC_ERR_DEVICE, "hipMemset(routes) failed: %s", hipGetErrorString(e));
  }
  h->pos = 0;
  h->has_prev_tok = false;
  return DEC_OK;
}

int32_t dec_position(const dec_handle* h) { return h ? h->pos : -1; }

int dec_read_kv(dec_handle* h, int32_t layer, int32_t seq, int32_t n_pos, uint16_t* host_k, uint16_t* host_v) {
  if (!h) return fail(nullptr, DEC_ERR_INVALID_ARG, "handle is NULL");
  const dec_model_desc& d = h->desc;
  if (layer < 0 || layer >= d.n_layers || seq < 0 || seq >= d.batch || n_pos < 0 || n_pos > d.max_ctx)
    return fail(&h->err, DEC_ERR_INVALID_ARG, "layer/seq/n_pos out of range");
  if (int rc0 = srv_stop(h)) return rc0;
  HIPCHK(h, &h->err, hipStreamSynchronize(h->stream));
  const size_t head = (size_t)d.max_ctx * d.head_dim;
  for (int kind = 0; kind < 2; ++kind) {
    uint16_t* dst = kind ? host_v : host_k;
    if (!dst) continue;
    for (int hh = 0; hh < d.n_heads; ++hh) {
      const uint16_t* src = h->P.kv + ((((size_t)layer * 2 + kind) * d.batch + seq) * d.n_heads + hh) * head;
      HIPCHK(h, &h->err, hipMemcpy(dst + (size_t)hh * n_pos * d.head_dim, src, (size_t)n_pos * d.head_dim * 2, hipMemcpyDeviceToHost));
    }
  }
  return DEC_OK;
}

int dec_read_routes(dec_handle* h, int32_t pos0, int32_t n_pos, int32_t* out_routes) {
  if (!h) return fail(nullptr, DEC_ERR_INVALID_ARG, "handle is NULL");
  const dec_model_desc& d = h->desc;
  if (!moe(d)) return fail(&h->err, DEC_ERR_STATE, "a dense model has no routing");
  if (pos0 < 0 || n_pos < 0 || (long long)pos0 + n_pos > d.max_ctx || (n_pos > 0 && !out_routes))
    return fail(&h->err, DEC_ERR_INVALID_ARG, "positions [%d, %d) outside [0, max_ctx) or NULL output", pos0, pos0 + n_pos);
  if (int rc0 = srv_stop(h)) return rc0;
  HIPCHK(h, &h->err, hipStreamSynchronize(h->stream));
  const size_t per_pos = (size_t)d.n_layers * d.top_k;
  if (n_pos > 0)
    HIPCHK(h, &h->err, hipMemcpy(out_routes, h->P.routes + (size_t)pos0 * per_pos, (size_t)n_pos * per_pos * 4,
                                 hipMemcpyDeviceToHost));
  return DEC_OK;
}

int dec_stream_ceiling(int32_t device, uint64_t bytes, int32_t reps, double* out_gbps) {
  if (!out_gbps) return fail(nullptr, DEC_ERR_INVALID_ARG, "out_gbps is NULL");
  const uint64_t MiB = 1ull << 20;
  if (bytes < 64 * MiB || bytes > 64 * 1024 * MiB) return fail(nullptr, DEC_ERR_INVALID_ARG, "bytes must be in [64 MiB, 64 GiB]");
  if (reps < 1 || reps > 100) return fail(nullptr, DEC_ERR_INVALID_ARG, "reps must be in [1, 100]");
  bytes = bytes / MiB * MiB;
  if (hipSetDevice(device) != hipSuccess) return fail(nullptr, DEC_ERR_NO_DEVICE, "hipSetDevice(%d) failed", device);
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1)
    return fail(nullptr, DEC_ERR_DEVICE, "compute unit count unavailable");
  const int grid = cus;   // one workgroup per compute unit, as the decode kernel
  void* buf = nullptr;
  uint32_t* out = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = DEC_OK;
  float ms = 0.f;
  if (hipMalloc(&buf, bytes) != hipSuccess) {
    rc = fail(nullptr, DEC_ERR_OOM, "hipMalloc(%llu) failed", (unsigned long long)bytes);
  } else if (hipMalloc(reinterpret_cast<void**>(&out), (size_t)grid * kThreads * 4) != hipSuccess) {
    rc = fail(nullptr, DEC_ERR_OOM, "hipMalloc(out) failed");
  } else {
    hipError_t e = hipMemset(buf, 0x3c, bytes);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) e = (hipError_t)kernel_stream_read(buf, bytes / 16, out, grid);   // untimed pass
    if (e == hipSuccess) e = hipEventRecord(e0, nullptr);
    for (int r = 0; r < reps && e == hipSuccess; ++r) e = (hipError_t)kernel_stream_read(buf, bytes / 16, out, grid);
    if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e != hipSuccess) rc = fail(nullptr, DEC_ERR_DEVICE, "stream ceiling run failed: %s", hipGetErrorString(e));
  }
  if (e0) hipEventDestroy(e0);
  if (e1) hipEventDestroy(e1);
  if (out) hipFree(out);
  if (buf) hipFree(buf);
  if (rc == DEC_OK) {
    if (ms <= 0.f) return fail(nullptr, DEC_ERR_DEVICE, "no elapsed time measured");
    *out_gbps = (double)bytes * reps / (ms * 1e-3) / 1e9;
  }
  return rc;
}

int dec_read_trace(dec_handle* h, uint64_t* host, int32_t* out_grid, int32_t* out_stride, double* out_hz) {
  if (!h) return fail(nullptr, DEC_ERR_INVALID_ARG, "handle is NULL");
  if (out_grid) *out_grid = h->grid;
  if (out_stride) *out_stride = kTraceStride;
  if (out_hz) *out_hz = h->wall_hz;
  if (!host) return DEC_OK;
  if (!h->P.trace) return fail(&h->err, DEC_ERR_STATE, "handle was created without DEC_DEBUG_TRACE");
  if (int rc0 = srv_stop(h)) return rc0;
  HIPCHK(h, &h->err, hipStreamSynchronize(h->stream));
  HIPCHK(h, &h->err, hipMemcpy(host, h->P.trace, (size_t)h->grid * kTraceStride * 8, hipMemcpyDeviceToHost));
  return DEC_OK;
}

void dec_free(dec_handle* h) {
  if (!h) return;
  (void)srv_stop(h);
  if (h->stream) (void)hipStreamSynchronize(h->stream);
  if (h->mail) (void)hipHostFree(h->mail);
  if (h->lg_host) (void)hipHostFree(h->lg_host);
  if (h->noalloc) g_scratch_held[h->device] = false;   // the fixed scratch array is free again
  if (h->own_arena && h->base) (void)hipFree(h->base);
  if (h->own_stream && h->stream) (void)hipStreamDestroy(h->stream);
  delete h;
}

const char* dec_last_error(const dec_handle* h) {
  if (h) return h->err.c_str();
  return g_err.c_str();
}

}  // extern "C"
#pragma GCC visibility pop
