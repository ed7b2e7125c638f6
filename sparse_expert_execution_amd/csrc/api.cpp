// api.cpp - C ABI entry points: argument checks, workspace carve-up, and the
// launches of the gfx950 kernels.  Declarations and contracts: include/moe.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/moe.h"
#include "hip_error.hpp"
#include "kernels.hpp"

namespace moe {

int hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return MOE_OK;
  return set_error(MOE_EHIP, "%s: %s (%s)", what, hipGetErrorName(err), hipGetErrorString(err));
}

}  // namespace moe

using moe::hip_status;
using moe::set_error;

namespace {
constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
}  // namespace


using moe::check_desc;
using moe::layout;

namespace {

struct PrefillWs {
  size_t xq_codes, xq_scales, chunk_counts, seg_start, tiles, sorted_pair, hq_codes, hq_scales,
      partial, total;
  int n_chunks, max_tiles, n_pairs;
};

PrefillWs prefill_ws(const moe_desc* d, int T) {
  PrefillWs w;
  const size_t H = d->hidden, I = d->inter, E = d->n_experts, k = d->top_k;
  w.n_pairs = (int)(T * k + (d->has_shared ? T : 0));
  w.n_chunks = (w.n_pairs + moe::kPrefillChunk - 1) / moe::kPrefillChunk;
  w.max_tiles = moe::prefill_max_tiles(T, (int)k, (int)E);
  // MXFP4 weights: MXFP4 copies of x and h; NVFP4: h in BF16 (x as given)
  const bool nv = d->wtype == MOE_WTYPE_NVFP4;
  size_t o = 0;
  w.xq_codes = o; o = align_up(o + (nv ? 0 : T * H / 2));
  w.xq_scales = o; o = align_up(o + (nv ? 0 : T * H / 32));
  w.chunk_counts = o; o = align_up(o + (size_t)w.n_chunks * (E + 1) * 4);
  w.seg_start = o; o = align_up(o + (E + 2) * 4);
  w.tiles = o; o = align_up(o + (1 + 2 * (size_t)w.max_tiles) * 4);
  w.sorted_pair = o; o = align_up(o + (size_t)w.n_pairs * 4);
  w.hq_codes = o; o = align_up(o + (size_t)w.n_pairs * (nv ? I * 2 : I / 2));
  w.hq_scales = o; o = align_up(o + (nv ? 0 : (size_t)w.n_pairs * I / 32));
  w.partial = o; o = align_up(o + (size_t)T * (k + 1) * H * 4);
  w.total = o;
  return w;
}

// route workspace: [0, 256) ticket counter, then router logits z [T][E].
// decode workspace: [0, 8192) counters and the launch generation, then
// kZCopies copies of z [T][E] and h [T*k + T][I] (8 bytes each: the fp32
// value and the launch generation it belongs to) and
// per-workgroup phase stamps (written only when timing is switched on).  The
// whole workspace must be zero before its first use; every call leaves the
// counters zero.
struct RouteWs {
  size_t z, h, st, total;
};
constexpr size_t kDecodeHeader = 8192;
RouteWs route_ws(const moe_desc* d, int T, bool decode) {
  RouteWs w;
  w.z = decode ? kDecodeHeader : kAlign;
  w.h = align_up(w.z + (decode ? moe::kZCopies * moe::decode_z_copy_bytes(T, d->n_experts)
                              : (size_t)T * d->n_experts * 4));
  w.st = decode ? align_up(w.h + (size_t)(T * d->top_k + T) * d->inter * 8) : w.h;
  w.total = decode ? w.st + moe::kDecodeStampBytes : w.h;
  return w;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_desc* desc, int32_t T, int32_t mode) {
  if (check_desc(desc)) return 0;
  if (T < 0) { set_error(MOE_EINVAL, "T < 0"); return 0; }
  switch (mode) {
    case MOE_MODE_ROUTE:
      return route_ws(desc, T, false).total;
    case MOE_MODE_DECODE:
      return route_ws(desc, T, true).total;
    case MOE_MODE_PREFILL:
      return prefill_ws(desc, T).total;
    default:
      set_error(MOE_EINVAL, "unknown mode %d", mode);
      return 0;
  }
}

int moe_route(const moe_desc* desc, const void* x, const void* w_router, int32_t T,
              int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream) {
  moe::ApiRange range_("moe_route");
  int st = check_desc(desc);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if (T < 0) return set_error(MOE_EINVAL, "T < 0");
  if (!x || !w_router || !ids || !w) return set_error(MOE_EINVAL, "null pointer");
  const RouteWs L = route_ws(desc, T, false);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return set_error(MOE_EWORKSPACE, "route workspace %zu < %zu bytes (or not 256-aligned)",
                     ws_bytes, L.total);
  if (!aligned(x, 16) || !aligned(w_router, 16))
    return set_error(MOE_EINVAL, "x and w_router must be 16-byte aligned");
  const int rf32 = desc->router_wtype == MOE_WTYPE_F32;
  uint8_t* b = static_cast<uint8_t*>(ws);
  float* z = reinterpret_cast<float*>(b + L.z);
  if (T <= MOE_DECODE_MAX_T && moe::route_small_supported(rf32, desc->hidden))
    return hip_status(moe::launch_route_small(x, w_router, rf32, T, desc->hidden,
                                              desc->n_experts, desc->top_k, desc->renorm_topk, z,
                                              reinterpret_cast<unsigned*>(b), ids, w,
                                              as_stream(stream)),
                      "moe_route");
  return hip_status(moe::launch_route_large(x, w_router, rf32, T, desc->hidden, desc->n_experts,
                                            desc->top_k, desc->renorm_topk, z, ids, w,
                                            as_stream(stream)),
                    "moe_route");
}

static int check_ffn_args(const moe_desc* desc, const void* x, int32_t T, const int32_t* ids,
                          const float* w, const void* slot_pool, const void* shared_expert,
                          float* y) {
  int st = check_desc(desc);
  if (st) return st;
  if (!x || !ids || !w || !slot_pool || !y) return set_error(MOE_EINVAL, "null pointer");
  if (desc->has_shared && !shared_expert)
    return set_error(MOE_EINVAL, "has_shared set but shared_expert is null");
  if (!desc->has_shared && shared_expert)
    return set_error(MOE_EINVAL, "shared_expert given but has_shared is 0");
  if (!aligned(x, 16) || !aligned(slot_pool, 256) || !aligned(y, 16) ||
      (shared_expert && !aligned(shared_expert, 256)))
    return set_error(MOE_EINVAL, "x, y need 16-byte and expert blocks 256-byte alignment");
  (void)T;
  return MOE_OK;
}

static int decode_impl(const moe_desc* desc, const void* x, const void* w_router, int32_t T,
                       int32_t* ids, float* w, const int32_t* slot_of_expert,
                       const void* slot_pool, const void* shared_expert, float* y, void* ws,
                       size_t ws_bytes, void* stream) {
  if (desc->top_k > 8)
    return set_error(MOE_EUNSUPPORTED, "decode supports top_k <= 8 (got %d)", desc->top_k);
  if (T < 0 || T > MOE_DECODE_MAX_T || T * desc->top_k > 1024)
    return set_error(MOE_EINVAL, "decode T %d outside [1, %d] or T*k > 1024", T, MOE_DECODE_MAX_T);
  if (!moe::decode_shape_supported(desc->wtype, desc->hidden, desc->inter))
    return set_error(MOE_EUNSUPPORTED, "decode shape H=%d I=%d not compiled", desc->hidden,
                     desc->inter);
  const RouteWs L = route_ws(desc, T, true);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return set_error(MOE_EWORKSPACE, "decode workspace %zu < %zu bytes (or not 256-aligned)",
                     ws_bytes, L.total);
  uint8_t* b = static_cast<uint8_t*>(ws);
  size_t off[6], bytes;
  layout(desc, off, &bytes);
  moe::DecodeLaunch f;
  f.x = x; f.w_router = w_router; f.router_f32 = desc->router_wtype == MOE_WTYPE_F32;
  f.renorm = desc->renorm_topk; f.ids = ids; f.w = w; f.slot_of = slot_of_expert;
  f.pool = slot_pool; f.shared = shared_expert;
  f.hdr = reinterpret_cast<unsigned*>(b);
  f.z = reinterpret_cast<uint64_t*>(b + L.z);
  f.zstride = (int64_t)(moe::decode_z_copy_bytes(T, desc->n_experts) / 8);
  f.h = reinterpret_cast<uint64_t*>(b + L.h);
  f.stamps = reinterpret_cast<unsigned long long*>(b + L.st);
  f.y = y; f.expert_bytes = (int64_t)bytes;
  for (int i = 0; i < 6; ++i) f.off[i] = (int64_t)off[i];
  f.goff = desc->wtype == MOE_WTYPE_NVFP4
               ? (int64_t)(off[5] + (size_t)desc->hidden * desc->inter / 16) : 0;
  f.H = desc->hidden; f.I = desc->inter; f.E = desc->n_experts; f.k = desc->top_k;
  f.wtype = desc->wtype;
  // launches of at most decode_max_tokens tokens, in stream order, the
  // batch split evenly over them
  const int H = desc->hidden, k = desc->top_k;
  const int cap = moe::decode_max_tokens(desc->wtype, H, desc->inter);
  const int n_launch = (T + cap - 1) / cap;
  const int per = (T + n_launch - 1) / n_launch;
  for (int t0 = 0; t0 < T; t0 += per) {
    f.T = T - t0 < per ? T - t0 : per;
    f.x = static_cast<const uint16_t*>(x) + (size_t)t0 * H;
    f.ids = ids + (size_t)t0 * k;
    f.w = w + (size_t)t0 * k;
    f.y = y + (size_t)t0 * H;
    const int st = hip_status(moe::launch_decode(f, as_stream(stream)),
                              w_router ? "moe_route_decode" : "moe_decode");
    if (st) return st;
  }
  return MOE_OK;
}

int32_t moe_decode_launch_tokens(const moe_desc* desc) {
  const int st = check_desc(desc);
  if (st) return st;
  if (!moe::decode_shape_supported(desc->wtype, desc->hidden, desc->inter))
    return set_error(MOE_EUNSUPPORTED, "decode shape H=%d I=%d not compiled", desc->hidden,
                     desc->inter);
  return moe::decode_max_tokens(desc->wtype, desc->hidden, desc->inter);
}

int moe_decode(const moe_desc* desc, const void* x, int32_t T, const int32_t* ids, const float* w,
               const int32_t* slot_of_expert, const void* slot_pool, const void* shared_expert,
               float* y, void* ws, size_t ws_bytes, void* stream) {
  moe::ApiRange range_("moe_decode");
  if (T == 0) return check_desc(desc);
  int st = check_ffn_args(desc, x, T, ids, w, slot_pool, shared_expert, y);
  if (st) return st;
  return decode_impl(desc, x, nullptr, T, const_cast<int32_t*>(ids), const_cast<float*>(w),
                     slot_of_expert, slot_pool, shared_expert, y, ws, ws_bytes, stream);
}

int moe_route_decode(const moe_desc* desc, const void* x, const void* w_router, int32_t T,
                     int32_t* ids, float* w, const int32_t* slot_of_expert,
                     const void* slot_pool, const void* shared_expert, float* y, void* ws,
                     size_t ws_bytes, void* stream) {
  moe::ApiRange range_("moe_route_decode");
  if (T == 0) return check_desc(desc);
  int st = check_ffn_args(desc, x, T, ids, w, slot_pool, shared_expert, y);
  if (st) return st;
  if (!w_router) return set_error(MOE_EINVAL, "w_router is null");
  if (!aligned(w_router, 16)) return set_error(MOE_EINVAL, "w_router must be 16-byte aligned");
  if (!moe::route_small_supported(desc->router_wtype == MOE_WTYPE_F32, desc->hidden))
    return set_error(MOE_EUNSUPPORTED, "hidden %d too wide for the decode router", desc->hidden);
  return decode_impl(desc, x, w_router, T, ids, w, slot_of_expert, slot_pool, shared_expert, y,
                     ws, ws_bytes, stream);
}

int moe_prefill(const moe_desc* desc, const void* x, int32_t T, const int32_t* ids, const float* w,
                const int32_t* slot_of_expert, const void* slot_pool, const void* shared_expert,
                float* y, void* ws, size_t ws_bytes, void* stream) {
  moe::ApiRange range_("moe_prefill");
  if (T == 0) return check_desc(desc);
  int st = check_ffn_args(desc, x, T, ids, w, slot_pool, shared_expert, y);
  if (st) return st;
  if (desc->wtype != MOE_WTYPE_MXFP4 && desc->wtype != MOE_WTYPE_NVFP4)
    return set_error(MOE_EUNSUPPORTED, "moe_prefill runs MXFP4 or NVFP4 expert weights");
  if (desc->hidden % 128 || desc->inter % 128)
    return set_error(MOE_EUNSUPPORTED, "moe_prefill needs hidden and inter multiples of 128");
  if (T < 0 || T > 65536) return set_error(MOE_EINVAL, "prefill T %d outside [1, 65536]", T);
  const PrefillWs L = prefill_ws(desc, T);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return set_error(MOE_EWORKSPACE, "prefill workspace %zu < %zu bytes", ws_bytes, L.total);
  uint8_t* b = static_cast<uint8_t*>(ws);
  moe::PrefillLaunch p;
  size_t off[6], bytes;
  layout(desc, off, &bytes);
  p.x = x; p.ids = ids; p.w = w; p.slot_of = slot_of_expert; p.pool = slot_pool;
  p.shared = shared_expert; p.y = y; p.expert_bytes = (int64_t)bytes;
  for (int i = 0; i < 6; ++i) p.off[i] = (int64_t)off[i];
  p.T = T; p.H = desc->hidden; p.I = desc->inter; p.E = desc->n_experts; p.k = desc->top_k;
  p.nvfp4 = desc->wtype == MOE_WTYPE_NVFP4;
  p.goff = p.nvfp4 ? (int64_t)(off[5] + (size_t)desc->hidden * desc->inter / 16) : 0;
  p.xq_codes = p.nvfp4 ? nullptr : b + L.xq_codes;
  p.xq_scales = p.nvfp4 ? nullptr : b + L.xq_scales;
  p.chunk_counts = reinterpret_cast<int32_t*>(b + L.chunk_counts);
  p.seg_start = reinterpret_cast<int32_t*>(b + L.seg_start);
  p.tiles = reinterpret_cast<int32_t*>(b + L.tiles);
  p.sorted_pair = reinterpret_cast<int32_t*>(b + L.sorted_pair);
  p.hq_codes = b + L.hq_codes;
  p.hq_scales = b + L.hq_scales;
  p.partial = reinterpret_cast<float*>(b + L.partial);
  p.n_chunks = L.n_chunks;
  p.max_tiles = L.max_tiles;
  return hip_status(moe::launch_prefill(p, as_stream(stream)), "moe_prefill");
}

int moe_debug_prefill_layout(const moe_desc* desc, int32_t T, int64_t out[5]) {
  int st = check_desc(desc);
  if (st) return st;
  if (!out || T < 1) return set_error(MOE_EINVAL, "bad argument");
  const PrefillWs L = prefill_ws(desc, T);
  out[0] = (int64_t)L.seg_start;
  out[1] = (int64_t)L.tiles;
  out[2] = (int64_t)L.sorted_pair;
  out[3] = L.max_tiles;
  out[4] = L.n_pairs;
  return MOE_OK;
}

int moe_merge_partials(const float* a, const float* b, float* y, size_t n, void* stream) {
  moe::ApiRange range_("moe_merge_partials");
  if (n == 0) return MOE_OK;
  if (!a || !b || !y) return set_error(MOE_EINVAL, "null pointer");
  return hip_status(moe::launch_merge(a, b, y, n, as_stream(stream)), "moe_merge_partials");
}

int moe_quantize_mxfp4(const float* src, int32_t rows, int32_t K, int64_t src_ld, uint8_t* codes,
                       uint8_t* scales, void* stream) {
  moe::ApiRange range_("moe_quantize_mxfp4");
  if (rows == 0) return MOE_OK;
  if (!src || !codes || !scales) return set_error(MOE_EINVAL, "null pointer");
  if (rows < 0 || K <= 0 || K % 32 || src_ld < K || src_ld % 4)
    return set_error(MOE_EINVAL, "bad shape rows=%d K=%d ld=%lld", rows, K, (long long)src_ld);
  if (!aligned(src, 16) || !aligned(codes, 16))
    return set_error(MOE_EINVAL, "src and codes must be 16-byte aligned");
  return hip_status(moe::launch_quantize_mxfp4(src, 0, rows, K, src_ld, codes, scales,
                                               as_stream(stream)),
                    "moe_quantize_mxfp4");
}

int moe_pack_expert(const moe_desc* desc, const void* gate, const void* up, const void* down,
                    int32_t src_type, void* dst, void* stream) {
  moe::ApiRange range_("moe_pack_expert");
  int st = check_desc(desc);
  if (st) return st;
  if (!gate || !up || !down || !dst) return set_error(MOE_EINVAL, "null pointer");
  if (src_type != MOE_WTYPE_F32 && src_type != MOE_WTYPE_BF16)
    return set_error(MOE_EUNSUPPORTED, "source type %d not supported", src_type);
  if (!aligned(gate, 16) || !aligned(up, 16) || !aligned(down, 16) || !aligned(dst, 256))
    return set_error(MOE_EINVAL, "sources need 16-byte and dst 256-byte alignment");
  size_t off[6], bytes;
  layout(desc, off, &bytes);
  const int H = desc->hidden, I = desc->inter;
  const int sb = src_type == MOE_WTYPE_BF16;
  uint8_t* b = static_cast<uint8_t*>(dst);
  hipStream_t s = as_stream(stream);
  hipError_t err;
  if (desc->wtype == MOE_WTYPE_BF16) {
    err = moe::launch_pack_bf16(gate, sb, I, H, reinterpret_cast<uint16_t*>(b + off[0]), s);
    if (err == hipSuccess)
      err = moe::launch_pack_bf16(up, sb, I, H, reinterpret_cast<uint16_t*>(b + off[1]), s);
    if (err == hipSuccess)
      err = moe::launch_pack_bf16(down, sb, H, I, reinterpret_cast<uint16_t*>(b + off[2]), s);
  } else if (desc->wtype == MOE_WTYPE_NVFP4) {
    float* gs = reinterpret_cast<float*>(b + off[5] + (size_t)H * I / 16);
    err = moe::launch_quantize_nvfp4(gate, sb, I, H, b + off[0], b + off[1], gs + 0, s);
    if (err == hipSuccess)
      err = moe::launch_quantize_nvfp4(up, sb, I, H, b + off[2], b + off[3], gs + 1, s);
    if (err == hipSuccess)
      err = moe::launch_quantize_nvfp4(down, sb, H, I, b + off[4], b + off[5], gs + 2, s);
  } else {
    err = moe::launch_quantize_mxfp4(gate, sb, I, H, H, b + off[0], b + off[1], s);
    if (err == hipSuccess)
      err = moe::launch_quantize_mxfp4(up, sb, I, H, H, b + off[2], b + off[3], s);
    if (err == hipSuccess)
      err = moe::launch_quantize_mxfp4(down, sb, H, I, I, b + off[4], b + off[5], s);
  }
  return hip_status(err, "moe_pack_expert");
}

int moe_debug_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t n_blocks,
                            float* out, void* stream) {
  if (n_blocks == 0) return MOE_OK;
  if (!codes || !scales || !out || n_blocks < 0) return set_error(MOE_EINVAL, "bad argument");
  if (!aligned(codes, 16) || !aligned(out, 16))
    return set_error(MOE_EINVAL, "codes and out must be 16-byte aligned");
  return hip_status(moe::launch_dequant_mxfp4(codes, scales, n_blocks, out, as_stream(stream)),
                    "moe_debug_dequant_mxfp4");
}

int moe_debug_dot_fp4(int32_t wtype, const uint8_t* codes, const uint8_t* scales,
                      const void* x, int64_t n_blocks, int32_t n_x, float* out, void* stream) {
  if (n_blocks == 0 || n_x == 0) return MOE_OK;
  if (wtype != MOE_WTYPE_MXFP4 && wtype != MOE_WTYPE_NVFP4)
    return set_error(MOE_EINVAL, "moe_debug_dot_fp4 takes MXFP4 or NVFP4 blocks");
  if (!codes || !scales || !x || !out || n_blocks < 0 || n_x < 0)
    return set_error(MOE_EINVAL, "bad argument");
  if (!aligned(codes, 16) || !aligned(x, 16))
    return set_error(MOE_EINVAL, "codes and x must be 16-byte aligned");
  return hip_status(moe::launch_dot_fp4(codes, scales, static_cast<const uint16_t*>(x), n_blocks,
                                        n_x, wtype == MOE_WTYPE_NVFP4, out, as_stream(stream)),
                    "moe_debug_dot_fp4");
}

int moe_decode_status(void* ws, size_t ws_bytes, int32_t* status, int32_t clear, void* stream) {
  if (!ws || ws_bytes < kDecodeHeader || !aligned(ws, 256))
    return set_error(MOE_EWORKSPACE, "decode status needs the decode workspace (>= %zu bytes)",
                     kDecodeHeader);
  if (!status && !clear) return MOE_OK;
  return hip_status(moe::launch_decode_status(static_cast<unsigned*>(ws), status, clear != 0,
                                              as_stream(stream)),
                    "moe_decode_status");
}

int moe_debug_mfma_fp4_tile(const uint8_t* a_codes, const uint8_t* a_scales,
                            const uint8_t* b_codes, const uint8_t* b_scales, float* out,
                            void* stream) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !out)
    return set_error(MOE_EINVAL, "null pointer");
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16))
    return set_error(MOE_EINVAL, "codes must be 16-byte aligned");
  return hip_status(moe::launch_mfma_fp4_tile(a_codes, a_scales, b_codes, b_scales, out,
                                              as_stream(stream)),
                    "moe_debug_mfma_fp4_tile");
}

int moe_debug_wave_scan(const int32_t* in, int32_t* out, int32_t n_waves, void* stream) {
  if (!in || !out || n_waves < 1) return set_error(MOE_EINVAL, "bad wave-scan arguments");
  return hip_status(moe::launch_wave_scan(in, out, n_waves, as_stream(stream)),
                    "moe_debug_wave_scan");
}

int moe_debug_read_probe(const void* buf, size_t bytes, int32_t blocks, uint32_t* out,
                         void* stream) {
  if (!buf || !out || blocks < 1 || !aligned(buf, 16))
    return set_error(MOE_EINVAL, "bad read-probe arguments");
  return hip_status(moe::launch_read_probe(buf, bytes, blocks, out, as_stream(stream)),
                    "moe_debug_read_probe");
}

}  // extern "C"
