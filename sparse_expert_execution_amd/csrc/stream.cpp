// stream.cpp - full-layer streaming of expert weights for prefill.
//
// A long prompt routes to nearly every expert of a layer, so prefill moves
// whole layers: with two full-layer buffers the next layer is copied over
// PCIe while the GPU computes the current one (explainx.ai guide, "Prefill:
// load almost every expert without idling the GPU"; futuresignalnews.com
// article, "2. Semantic-Aware Caching").  With one buffer the
// copy of a layer and its compute run one after the other (the pages'
// ablation).  A layer's block in the pinned host pool is copied with one
// hipMemcpyAsync on a copy stream; HIP events order it after the buffer's
// previous reader and before the compute stream's use.
#include <hip/hip_runtime.h>

#include <new>

#include "../../include/moe.h"
#include "hip_error.hpp"

using moe::hip_status;
using moe::set_error;

struct moe_layer_stream {
  const uint8_t* host_pool = nullptr;
  int32_t n_layers = 0;
  size_t layer_bytes = 0;
  int nb = 0;
  uint8_t* buf[2] = {nullptr, nullptr};
  int32_t held[2] = {-1, -1};        // layer a buffer holds (or is receiving)
  bool released[2] = {true, true};   // its holder's work has been released
  bool free_recorded[2] = {false, false};
  hipEvent_t copy_done[2] = {nullptr, nullptr};
  hipEvent_t free_ev[2] = {nullptr, nullptr};
};

namespace {

// copy `layer` into buffer b after the buffer's last release
int issue_copy(moe_layer_stream* s, int32_t layer, int b, hipStream_t copy) {
  if (!s->released[b])
    return set_error(MOE_ECACHE, "buffer of layer %d is still in use (release it first)",
                     s->held[b]);
  hipError_t err = hipSuccess;
  if (s->free_recorded[b]) err = hipStreamWaitEvent(copy, s->free_ev[b], 0);
  if (err == hipSuccess)
    err = hipMemcpyAsync(s->buf[b], s->host_pool + (size_t)layer * s->layer_bytes,
                         s->layer_bytes, hipMemcpyHostToDevice, copy);
  if (err == hipSuccess) err = hipEventRecord(s->copy_done[b], copy);
  if (err != hipSuccess) {
    s->held[b] = -1;
    return hip_status(err, "moe_layer_stream copy");
  }
  s->held[b] = layer;
  s->released[b] = false;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_stream_create(moe_layer_stream** out, const void* host_pool, int32_t n_layers,
                            size_t layer_bytes, void* dev_buf0, void* dev_buf1) {
  if (!out) return set_error(MOE_EINVAL, "null output");
  *out = nullptr;
  if (!host_pool || !dev_buf0 || n_layers < 1 || layer_bytes == 0)
    return set_error(MOE_EINVAL, "null pool/buffer, n_layers < 1 or layer_bytes 0");
  if (dev_buf1) {
    const uint8_t* a = static_cast<const uint8_t*>(dev_buf0);
    const uint8_t* b = static_cast<const uint8_t*>(dev_buf1);
    if (a < b + layer_bytes && b < a + layer_bytes)
      return set_error(MOE_EINVAL, "the two layer buffers overlap");
  }
  moe_layer_stream* s = new (std::nothrow) moe_layer_stream;
  if (!s) return set_error(MOE_EINVAL, "out of host memory");
  s->host_pool = static_cast<const uint8_t*>(host_pool);
  s->n_layers = n_layers;
  s->layer_bytes = layer_bytes;
  s->nb = dev_buf1 ? 2 : 1;
  s->buf[0] = static_cast<uint8_t*>(dev_buf0);
  s->buf[1] = static_cast<uint8_t*>(dev_buf1);
  hipError_t err = hipSuccess;
  for (int b = 0; b < s->nb && err == hipSuccess; ++b) {
    err = hipEventCreateWithFlags(&s->copy_done[b], hipEventDisableTiming);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&s->free_ev[b], hipEventDisableTiming);
  }
  if (err != hipSuccess) {
    moe_layer_stream_destroy(s);
    return hip_status(err, "moe_layer_stream_create");
  }
  *out = s;
  return MOE_OK;
}

void moe_layer_stream_destroy(moe_layer_stream* s) {
  if (!s) return;
  for (int b = 0; b < 2; ++b) {
    if (s->copy_done[b]) (void)hipEventDestroy(s->copy_done[b]);
    if (s->free_ev[b]) (void)hipEventDestroy(s->free_ev[b]);
  }
  delete s;
}

int moe_layer_stream_acquire(moe_layer_stream* s, int32_t layer, void* copy_stream,
                             void* compute_stream, void** dev_layer) {
  moe::ApiRange range_("moe_layer_stream_acquire");
  if (!s || !dev_layer) return set_error(MOE_EINVAL, "null pointer");
  if (layer < 0 || layer >= s->n_layers)
    return set_error(MOE_EINVAL, "layer %d out of range", layer);
  hipStream_t copy = static_cast<hipStream_t>(copy_stream);
  hipStream_t comp = static_cast<hipStream_t>(compute_stream);
  const int b = layer % s->nb;
  if (s->held[b] != layer) {
    const int st = issue_copy(s, layer, b, copy);
    if (st) return st;
  }
  s->released[b] = false;                  // in use until its next release
  hipError_t err = hipStreamWaitEvent(comp, s->copy_done[b], 0);
  if (err != hipSuccess) return hip_status(err, "moe_layer_stream_acquire");
  // double buffering: the next layer starts streaming now, into the buffer
  // whose layer has been released (else it waits for the next acquire)
  if (s->nb == 2 && layer + 1 < s->n_layers) {
    const int b2 = (layer + 1) % 2;
    if (s->held[b2] != layer + 1 && s->released[b2]) {
      const int st = issue_copy(s, layer + 1, b2, copy);
      if (st) return st;
    }
  }
  *dev_layer = s->buf[b];
  return MOE_OK;
}

int moe_layer_stream_release(moe_layer_stream* s, int32_t layer, void* compute_stream) {
  moe::ApiRange range_("moe_layer_stream_release");
  if (!s) return set_error(MOE_EINVAL, "null stream object");
  if (layer < 0 || layer >= s->n_layers)
    return set_error(MOE_EINVAL, "layer %d out of range", layer);
  const int b = layer % s->nb;
  if (s->held[b] != layer || s->released[b])
    return set_error(MOE_ECACHE, "layer %d is not held", layer);
  hipError_t err = hipEventRecord(s->free_ev[b], static_cast<hipStream_t>(compute_stream));
  if (err != hipSuccess) return hip_status(err, "moe_layer_stream_release");
  s->free_recorded[b] = true;
  s->released[b] = true;
  return MOE_OK;
}

}  // extern "C"
