// C entry points: argument validation on the host, then kernel launch on the
// caller's stream. Nothing here allocates or synchronises.
#include <limits.h>

#include <mutex>
#include <vector>

#include "../../include/aqlm.h"
#include "aqlm_internal.hpp"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validate the layer descriptor and fill the internal description.
int check_layer(const aqlm_layer *layer, aqlm::LayerDesc *d) {
  if (!layer) return AQLM_ERR_NULL;
  if (!layer->codes || !layer->codebooks || !layer->scales) return AQLM_ERR_NULL;
  const int M = layer->num_codebooks, B = layer->nbits, g = layer->group_size;
  aqlm::Scheme s;
  if (M == 2 && B == 8 && g == 8)
    s = aqlm::Scheme::k2x8;
  else if (M == 1 && B == 16 && g == 8)
    s = aqlm::Scheme::k1x16;
  else if (M == 1 && B == 16 && g == 16)
    s = aqlm::Scheme::k1x16g16;
  else if (M >= 1 && M <= 8 && B >= 8 && B <= 16 && (g == 8 || g == 16))
    s = aqlm::Scheme::kGeneral;
  else
    return AQLM_ERR_SCHEME;
  if (layer->flags != 0 && layer->flags != AQLM_CODES_PACKED) return AQLM_ERR_SHAPE;
  if (layer->out_features < 1 || layer->in_features < 1) return AQLM_ERR_SHAPE;
  if (layer->in_features % g) return AQLM_ERR_SHAPE;
  // Kernels index rows and columns with 32-bit integers.
  if (layer->out_features > INT_MAX / 2 || layer->in_features > INT_MAX / 2) return AQLM_ERR_SHAPE;
  // bit-packed streams are read with 32-bit byte offsets
  const bool packed = layer->flags == AQLM_CODES_PACKED;
  if (packed && layer->out_features * (layer->in_features / g) >= ((int64_t)1 << 35) / (M * B))
    return AQLM_ERR_SHAPE;
  if (!aligned16(layer->codes) || !aligned16(layer->codebooks) || !aligned16(layer->scales))
    return AQLM_ERR_ALIGN;
  d->out = layer->out_features;
  d->in = layer->in_features;
  d->groups = layer->in_features / g;
  d->scheme = s;
  d->M = M;
  d->B = B;
  d->g = g;
  d->packed = packed;
  d->codes = layer->codes;
  d->books = layer->codebooks;
  d->scales = layer->scales;
  return AQLM_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? AQLM_OK : AQLM_ERR_HIP; }

// Validation shared by the grouped GEMV entry points: fills d; checks x and
// y unless check_io is false.
int check_layers(const aqlm_layer *layers, const uint16_t *const *x, uint16_t *const *y,
                 int32_t num_layers, int64_t batch, std::vector<aqlm::LayerDesc> *d,
                 bool check_io) {
  if (num_layers < 0 || num_layers > 4096) return AQLM_ERR_SHAPE;
  if (batch < 0 || batch > 8) return AQLM_ERR_BATCH;
  if (num_layers == 0 || batch == 0) return AQLM_OK;
  if (!layers) return AQLM_ERR_NULL;
  if (check_io && (!x || !y)) return AQLM_ERR_NULL;
  d->resize(num_layers);
  for (int i = 0; i < num_layers; ++i) {
    const int st = check_layer(&layers[i], &(*d)[i]);
    if (st != AQLM_OK) return st;
    if (!check_io) continue;
    if (!x[i] || !y[i]) return AQLM_ERR_NULL;
    if (!aligned16(x[i]) || !aligned16(y[i])) return AQLM_ERR_ALIGN;
  }
  return AQLM_OK;
}

}  // namespace

// Scratch memory of aqlm_gemm_noalloc: a static device array, one copy per GPU
// (created when the library's code is loaded on that device, kept until the
// process ends). In host code `scratch` is only a handle: its device address
// on each GPU comes from hipGetSymbolAddress, called once per device with
// that device current, and only that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[AQLM_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices];  // device address of `scratch` per device, or null

// The current device's scratch address (looked up on the first call there).
int scratch_address(void **out) {
  *out = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return AQLM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return AQLM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return AQLM_OK;
}

}  // namespace

extern "C" {

int aqlm_abi_version(void) { return AQLM_ABI_VERSION; }

const char *aqlm_status_string(int status) {
  switch (status) {
    case AQLM_OK: return "ok";
    case AQLM_ERR_NULL: return "a required pointer is NULL";
    case AQLM_ERR_SHAPE: return "invalid shape: need out >= 1, in >= 1, in % group_size == 0, "
                                "sizes below 2^30 and flags 0 or AQLM_CODES_PACKED";
    case AQLM_ERR_SCHEME: return "unsupported scheme: need 1 <= M <= 8 codebooks, 8 <= B <= 16 "
                                 "code bits and group size 8 or 16";
    case AQLM_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case AQLM_ERR_BATCH: return "batch outside the entry point's range";
    case AQLM_ERR_HIP: return "the HIP runtime reported an error";
    case AQLM_ERR_WORKSPACE: return "the workspace is smaller than aqlm_gemm_workspace_size";
    case AQLM_ERR_SCRATCH: return "the call needs more scratch memory than the library's static "
                                  "scratch array holds (AQLM_STATIC_SCRATCH_BYTES = 64 MiB); "
                                  "use aqlm_gemm_ws with a workspace or aqlm_gemm";
    default: return "unknown status";
  }
}

int aqlm_dequant(const aqlm_layer *layer, uint16_t *W, void *stream) {
  aqlm::LayerDesc d;
  const int st = check_layer(layer, &d);
  if (st != AQLM_OK) return st;
  if (!W) return AQLM_ERR_NULL;
  if (!aligned16(W)) return AQLM_ERR_ALIGN;
  return from_hip(aqlm::launch_dequant(d, W, static_cast<hipStream_t>(stream)));
}

int aqlm_gemv(const aqlm_layer *layer, const uint16_t *x, int64_t batch, uint16_t *y,
              void *stream) {
  aqlm::LayerDesc d;
  const int st = check_layer(layer, &d);
  if (st != AQLM_OK) return st;
  if (batch < 0 || batch > 8) return AQLM_ERR_BATCH;
  if (batch == 0) return AQLM_OK;
  if (!x || !y) return AQLM_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return AQLM_ERR_ALIGN;
  return from_hip(aqlm::launch_gemv(d, x, (int)batch, y, static_cast<hipStream_t>(stream)));
}

int aqlm_gemv_batched(const aqlm_layer *layers, const uint16_t *const *x, uint16_t *const *y,
                      int32_t num_layers, int64_t batch, void *stream) {
  std::vector<aqlm::LayerDesc> d;
  const int st = check_layers(layers, x, y, num_layers, batch, &d, true);
  if (st != AQLM_OK || num_layers == 0 || batch == 0) return st;
  return from_hip(aqlm::launch_gemv_batched(d.data(), x, y, num_layers, (int)batch,
                                            static_cast<hipStream_t>(stream)));
}

int aqlm_gemv_workspace_size(const aqlm_layer *layers, int32_t num_layers, int64_t batch,
                             int64_t *bytes) {
  if (!bytes) return AQLM_ERR_NULL;
  *bytes = 0;
  std::vector<aqlm::LayerDesc> d;
  const int st = check_layers(layers, nullptr, nullptr, num_layers, batch, &d, false);
  if (st != AQLM_OK) return st;
  if (num_layers == 0 || batch == 0) return AQLM_OK;
  *bytes = aqlm::gemv_ws_bytes(d.data(), num_layers, (int)batch);
  return AQLM_OK;
}

int aqlm_gemv_ws(const aqlm_layer *layers, const uint16_t *const *x, uint16_t *const *y,
                 int32_t num_layers, int64_t batch, void *workspace, int64_t workspace_bytes,
                 void *stream) {
  std::vector<aqlm::LayerDesc> d;
  const int st = check_layers(layers, x, y, num_layers, batch, &d, true);
  if (st != AQLM_OK) return st;
  if (num_layers == 0 || batch == 0) return AQLM_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t need = aqlm::gemv_ws_bytes(d.data(), num_layers, (int)batch);
  if (need == 0) return from_hip(aqlm::launch_gemv_batched(d.data(), x, y, num_layers, (int)batch, s));
  if (!workspace) return AQLM_ERR_NULL;
  if (!aligned16(workspace)) return AQLM_ERR_ALIGN;
  if (workspace_bytes < need) return AQLM_ERR_WORKSPACE;
  return from_hip(aqlm::launch_gemv_batched_ws(d.data(), x, y, num_layers, (int)batch, workspace, s));
}

namespace {
// batch range of the GEMM entry points (grid.y holds the activation-row tiles)
bool gemm_batch_ok(int64_t batch) {
  return batch >= 0 && batch <= (int64_t)INT_MAX / 2 && (batch + 63) / 64 <= 65535;
}
}  // namespace

int aqlm_gemm(const aqlm_layer *layer, const uint16_t *x, int64_t batch, uint16_t *y,
              void *stream) {
  aqlm::LayerDesc d;
  const int st = check_layer(layer, &d);
  if (st != AQLM_OK) return st;
  if (!gemm_batch_ok(batch)) return AQLM_ERR_BATCH;
  if (batch == 0) return AQLM_OK;
  if (!x || !y) return AQLM_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return AQLM_ERR_ALIGN;
  return from_hip(aqlm::launch_gemm(d, x, batch, y, static_cast<hipStream_t>(stream)));
}

int aqlm_gemm_workspace_size(const aqlm_layer *layer, int64_t batch, int64_t *bytes) {
  if (!bytes) return AQLM_ERR_NULL;
  *bytes = 0;
  aqlm::LayerDesc d;
  const int st = check_layer(layer, &d);
  if (st != AQLM_OK) return st;
  if (!gemm_batch_ok(batch)) return AQLM_ERR_BATCH;
  if (batch > 0) *bytes = aqlm::gemm_ws_bytes(d, batch);
  return AQLM_OK;
}

int aqlm_gemm_ws(const aqlm_layer *layer, const uint16_t *x, int64_t batch, uint16_t *y,
                 void *workspace, int64_t workspace_bytes, void *stream) {
  aqlm::LayerDesc d;
  const int st = check_layer(layer, &d);
  if (st != AQLM_OK) return st;
  if (!gemm_batch_ok(batch)) return AQLM_ERR_BATCH;
  if (batch == 0) return AQLM_OK;
  if (!x || !y) return AQLM_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return AQLM_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t need = aqlm::gemm_ws_bytes(d, batch);
  if (need == 0) return from_hip(aqlm::launch_gemm(d, x, batch, y, s));
  if (!workspace) return AQLM_ERR_NULL;
  if (!aligned16(workspace)) return AQLM_ERR_ALIGN;
  if (workspace_bytes < need) return AQLM_ERR_WORKSPACE;
  return from_hip(aqlm::launch_gemm_ws(d, x, batch, y, workspace, s));
}

int aqlm_gemm_noalloc(const aqlm_layer *layer, const uint16_t *x, int64_t batch, uint16_t *y,
                      void *stream) {
  aqlm::LayerDesc d;
  const int st = check_layer(layer, &d);
  if (st != AQLM_OK) return st;
  if (!gemm_batch_ok(batch)) return AQLM_ERR_BATCH;
  if (batch == 0) return AQLM_OK;
  if (!x || !y) return AQLM_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return AQLM_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t need = aqlm::gemm_ws_bytes(d, batch);
  if (need == 0) return from_hip(aqlm::launch_gemm(d, x, batch, y, s));
  if (need > AQLM_STATIC_SCRATCH_BYTES) return AQLM_ERR_SCRATCH;
  void *ws = nullptr;
  const int sst = scratch_address(&ws);
  if (sst != AQLM_OK) return sst;
  return from_hip(aqlm::launch_gemm_ws(d, x, batch, y, ws, s));
}

}  // extern "C"
