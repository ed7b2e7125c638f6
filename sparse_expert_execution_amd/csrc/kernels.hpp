// kernels.hpp - host-side launchers of the gfx950 kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct DecodeLaunch {
  const void* x;
  const void* w_router;   // null: ids / w are inputs
  int router_f32, renorm;
  int32_t* ids;
  float* w;
  const int32_t* slot_of;
  const void* pool;
  const void* shared;
  unsigned* hdr;          // counter header (zero before first use)
  uint64_t* z;            // kZCopies copies of [T][E] generation-tagged logits
  int64_t zstride;        // uint64 words from one copy to the next
  uint64_t* h;            // [T*k + T][I] generation-tagged h
  unsigned long long* stamps;  // [kMaxWorkgroups][16] phase stamps (timing only)
  float* y;
  int64_t expert_bytes;
  int64_t off[6];
  int64_t goff;           // NVFP4: offset of the three fp32 matrix scales, else 0
  int T, H, I, E, k, wtype;
};

struct PrefillLaunch {
  const void* x;
  const int32_t* ids;
  const float* w;
  const int32_t* slot_of;
  const void* pool;
  const void* shared;
  float* y;
  int64_t expert_bytes;
  int64_t off[6];
  int T, H, I, E, k;
  // workspace carve-up
  uint8_t* xq_codes;     // [T][H/2]
  uint8_t* xq_scales;    // [T][H/32]
  int32_t* chunk_counts; // [n_chunks][E+1]
  int32_t* seg_start;    // [E+2]
  int32_t* tiles;        // [2 * max_tiles + 1]: n_tiles, then (bin, row0) pairs
  int32_t* sorted_pair;  // [n_pairs]
  uint8_t* hq_codes;     // [n_pairs][I/2]   (sorted order); NVFP4: BF16 h [n_pairs][I]
  uint8_t* hq_scales;    // [n_pairs][I/32]; NVFP4: unused
  float* partial;        // [T][k+1][H]
  int nvfp4;             // weights NVFP4 (x not quantised, BF16 GEMMs)
  int64_t goff;          // NVFP4: offset of the three fp32 matrix scales
  int n_chunks, max_tiles;
};

// prefill GEMMs for NVFP4 weights (BF16 matrix cores); the sort is shared
struct NvPrefillArgs {
  const int32_t* slot_of;
  const uint8_t* pool;
  const uint8_t* shared;
  int64_t expert_bytes;
  int64_t off[6];
  int64_t goff;          // offset of the gate, up, down fp32 matrix scales
  int T, H, I, E, k;
  const int32_t* seg_start;
  const int32_t* tiles;
  const int32_t* sorted_pair;
  const uint16_t* x;     // [T][H] bf16
  uint16_t* hb;          // [n_pairs][I] bf16 h, sorted order
  float* partial;        // [T][k+1][H] per-pair outputs
};
hipError_t launch_prefill_nvfp4_gemms(const NvPrefillArgs& a, int max_tiles, hipStream_t st);

// router alone: small T (one wave per expert row, the last workgroup ranks),
// large T (tiled logits + one wave per token)
bool route_small_supported(int router_f32, int H);
hipError_t launch_route_small(const void* x, const void* w_router, int router_f32, int T, int H,
                              int E, int k, int renorm, float* z, unsigned* ticket, int32_t* ids,
                              float* w, hipStream_t st);
hipError_t launch_route_large(const void* x, const void* w_router, int router_f32, int T,
                              int H, int E, int k, int renorm, float* logits, int32_t* ids,
                              float* w, hipStream_t st);

// per-workgroup phase stamps at the end of the decode workspace
constexpr size_t kDecodeStampBytes = 1024 * 16 * 8;
// copies of the decode logits (each read by every kZCopies-th workgroup)
constexpr int kZCopies = 64;
// bytes of one copy: [T][E] uint64, rounded to 4 KB, plus 256 B so that the
// copies start at different offsets within a page
inline size_t decode_z_copy_bytes(int T, int E) {
  return (((size_t)T * E * 8 + 4095) & ~(size_t)4095) + 256;
}

// decode: router (optional) + experts + combine in one kernel, at most
// decode_max_tokens(H) tokens per launch
bool decode_shape_supported(int wtype, int H, int I);
int decode_max_tokens(int wtype, int H, int I);
hipError_t launch_decode(const DecodeLaunch& f, hipStream_t st);

// prefill
constexpr int kPrefillChunk = 256;   // pairs per sort chunk
constexpr int kPrefillMT = 128;      // rows per M tile
int prefill_max_tiles(int T, int k, int E);
hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t st);

// formats / merge
hipError_t launch_quantize_mxfp4(const void* src, int src_bf16, int rows, int K, int64_t ld,
                                 uint8_t* codes, uint8_t* scales, hipStream_t st);
// NVFP4: codes [rows][K/2], E4M3 scales [rows][K/16], fp32 matrix scale at g
hipError_t launch_quantize_nvfp4(const void* src, int src_bf16, int rows, int K, uint8_t* codes,
                                 uint8_t* scales, float* g, hipStream_t st);
hipError_t launch_pack_bf16(const void* src, int src_bf16, int rows, int K, uint16_t* dst,
                            hipStream_t st);
hipError_t launch_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales,
                                int64_t n_blocks, float* out, hipStream_t st);
// test hook: per (block, x vector) the decode gate/up block step (MXFP4 or NVFP4)
hipError_t launch_dot_fp4(const uint8_t* codes, const uint8_t* scales, const uint16_t* x,
                          int64_t n_blocks, int n_x, int nvfp4, float* out, hipStream_t st);
// decode header word 32 (a wait expired) to out, optionally cleared
hipError_t launch_decode_status(unsigned* hdr, int32_t* out, int clear, hipStream_t st);
hipError_t launch_merge(const float* a, const float* b, float* y, size_t n,
                        hipStream_t st);
hipError_t launch_mfma_fp4_tile(const uint8_t* a_codes, const uint8_t* a_scales,
                                const uint8_t* b_codes, const uint8_t* b_scales,
                                float* out, hipStream_t st);

hipError_t launch_wave_scan(const int32_t* in, int32_t* out, int n_waves, hipStream_t st);
hipError_t launch_read_probe(const void* src, size_t bytes, int blocks, uint32_t* out,
                             hipStream_t st);

// cache
hipError_t launch_fill_i32(int32_t* dst, int32_t value, int64_t n, hipStream_t st);

}  // namespace moe
