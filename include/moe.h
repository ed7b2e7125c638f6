/*
 * moe.h - C ABI of the routed Mixture-of-Experts layer for MI355X (gfx950).
 *
 * The layer this library computes is the sparse expert execution the
 * FreeToken pages describe: each token is routed to a few of many experts,
 * only those experts run, and the layer output is the sum of their weighted
 * partial results ("FreeToken 753b Model Explained", section of the same
 * name).  Expert weights are reached through an expert-cache slot table; a
 * global LRU cache in GPU memory is filled from a pinned host expert pool;
 * the partial sums of two disjoint expert subsets merge exactly
 * (explainx.ai guide, "Decode: decide whether to move an expert or compute
 * where it lives"; futuresignalnews.com article, "1. Bandwidth-Adaptive
 * Execution (The q* Policy)" and "2. Semantic-Aware Caching").
 *
 * Conventions for every call
 *   - Return value: MOE_OK (0) or a negative MOE_E* status; nothing aborts or
 *     throws across this boundary.  moe_last_error() returns a thread-local
 *     text for the last failing call on the calling thread.
 *   - Pointers named d_* or documented "device" are device memory of the
 *     current HIP device; "host" pointers are CPU memory.  The caller owns
 *     every buffer; no call keeps a pointer past its return except the cache
 *     object (see moe_cache_create).
 *   - Device work is enqueued on the caller's stream (a hipStream_t passed as
 *     void*; NULL = the null stream) and the call returns without
 *     synchronising.  A fault inside a kernel surfaces at the caller's next
 *     synchronisation, not as this call's status.
 *   - No call allocates device memory.  Scratch comes from a caller-provided
 *     workspace sized by moe_workspace_bytes().
 *   - Stateless calls are reentrant; a moe_planner / moe_cache object must
 *     not be used from two threads at once.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK 0
#define MOE_EINVAL (-1)       /* bad argument: null pointer, size, shape     */
#define MOE_EUNSUPPORTED (-2) /* weight type / shape / device not supported  */
#define MOE_EHIP (-3)         /* HIP runtime error (text in moe_last_error)  */
#define MOE_EWORKSPACE (-4)   /* workspace missing or too small              */
#define MOE_ECACHE (-5)       /* cache: invalid plan or not enough slots     */

/* ---- formats ----------------------------------------------------------- */
/* Expert / router weight formats.
 *   F32   : IEEE binary32 (router only).
 *   BF16  : bfloat16 (upper half of binary32), round-to-nearest-even.
 *   MXFP4 : OCP MX FP4: 4-bit e2m1 codes, two per byte (element 2j in the low
 *           nibble of byte j), plus one e8m0 scale byte (2^(s-127)) per 32
 *           consecutive elements along the reduction axis K.  The pages list
 *           MXFP4 among the engine's expert formats ("FreeToken 753b Model
 *           Explained", "Performance Benchmarks and Model Fit") without its
 *           bit layout; the OCP MX v1.0 definitions are used. */
#define MOE_WTYPE_F32 0
#define MOE_WTYPE_BF16 1
#define MOE_WTYPE_MXFP4 2
/* NVFP4: e2m1 codes [rows][K/2] (low nibble first), one OCP E4M3FN scale per
 * 16 elements [rows][K/16], one fp32 scale per matrix; value = e2m1 * E4M3 *
 * fp32 scale.  The pages name it for their GLM-5.2 and laptop builds
 * ("FreeToken 753b Model Explained", "Performance Benchmarks and Model
 * Fit").  Decode, prefill and the host expert kernel take it; CDNA4's scaled
 * FP4 matrix instructions take a power-of-two scale per 32 elements, so the
 * NVFP4 prefill runs on the BF16 matrix cores (see moe_prefill). */
#define MOE_WTYPE_NVFP4 3

/* Layer description.  hidden (H) and inter (I) must be multiples of 32
 * (MXFP4 blocks) and of 8 (BF16 16-byte vectors); 1 <= top_k <= n_experts
 * <= 1024. */
typedef struct moe_desc {
  int32_t hidden;       /* H: token width                                    */
  int32_t inter;        /* I: expert SwiGLU intermediate width               */
  int32_t n_experts;    /* E: routed experts                                 */
  int32_t top_k;        /* k: experts per token                              */
  int32_t has_shared;   /* 1: a shared expert also runs on every token, w=1  */
  int32_t renorm_topk;  /* 1: divide the k gate weights by their sum         */
  int32_t wtype;        /* expert weights: MOE_WTYPE_BF16, _MXFP4 or _NVFP4  */
  int32_t router_wtype; /* router weights: MOE_WTYPE_F32 or MOE_WTYPE_BF16   */
} moe_desc;

/* One expert is one contiguous block of moe_expert_layout()'s *bytes, laid
 * out identically in the pinned host pool and in a device slot (the pages'
 * direct host loading into the final layout, "FreeToken 753b Model
 * Explained", "How MoE Paging and Caching Work").  Sections, in order:
 *   BF16 : [0] gate [I][H], [1] up [I][H], [2] down [H][I]   (row-major,
 *          K contiguous); offsets[3..5] = 0.
 *   MXFP4: [0] gate codes [I][H/2], [1] gate scales [I][H/32],
 *          [2] up codes [I][H/2],   [3] up scales [I][H/32],
 *          [4] down codes [H][I/2], [5] down scales [H][I/32].
 *   NVFP4: as MXFP4 with scales [rows][K/16] (E4M3), followed at offset
 *          offsets[5] + H*I/16 by the fp32 scales of gate, up and down.
 * Section offsets are 16-byte aligned; *bytes is a multiple of 256.
 * moe_pack_expert writes this layout.
 * Returns MOE_EINVAL for a bad descriptor. */
int moe_expert_layout(const moe_desc* desc, size_t offsets[6], size_t* bytes);

/* Workspace bytes a call needs (0 if none).  mode: 0 = moe_route,
 * 1 = moe_decode / moe_route_decode, 2 = moe_prefill, for T tokens.  Returns
 * 0 and sets the error text for an invalid descriptor or T.  A route
 * workspace starts with a 256-byte counter header that must be zero before
 * its first use; every call leaves it zero again.  A decode workspace must be
 * zero as a whole before its first use (its 8 KB header holds counters, which
 * every call leaves zero, and the generation of the last launch, against which
 * the logits the kernel hands between workgroups are tagged).  A workspace
 * must not be used by two calls that can run concurrently.  Decode header
 * word 32 (uint32) is set to 1 if a wait inside the kernel expired (only
 * possible on an oversubscribed device); setting word 64 to non-zero makes
 * the kernel record phase timestamps (100 MHz clock, uint64) from word 1152
 * on and per workgroup at the end of the workspace. */
#define MOE_MODE_ROUTE 0
#define MOE_MODE_DECODE 1
#define MOE_MODE_PREFILL 2
size_t moe_workspace_bytes(const moe_desc* desc, int32_t T, int32_t mode);

/* Largest T moe_decode accepts (larger batches go through moe_prefill). */
#define MOE_DECODE_MAX_T 64

/* ---- router ------------------------------------------------------------ */
/* moe_route: z = W_r x (fp32 accumulation of exact products), p = softmax(z)
 * over all E experts (fp32), ids = the top_k experts by p in descending order
 * (ties to the lower id), w = p[ids] (divided by their sum if renorm_topk).
 * Routing picks a few experts per token and layer ("FreeToken 753b Model
 * Explained"); the gate function is not on the pages, softmax then top-k is
 * the reading used.
 *   x        device, [T][H] BF16 row-major
 *   w_router device, [E][H] in desc->router_wtype
 *   ids      device out, [T][k] int32
 *   w        device out, [T][k] float
 *   ws       device workspace of moe_workspace_bytes(desc, T, MOE_MODE_ROUTE)
 * T >= 1 (T == 0 is a no-op returning MOE_OK). */
int moe_route(const moe_desc* desc, const void* x, const void* w_router,
              int32_t T, int32_t* ids, float* w, void* ws, size_t ws_bytes,
              void* stream);

/* ---- expert FFNs + weighted combine ------------------------------------ */
/* moe_decode: y[t] = sum over j of w[t][j] * FFN_{ids[t][j]}(x[t])
 *                    (+ FFN_shared(x[t]) when desc->has_shared),
 * FFN_e(x) = W_down (silu(W_gate x) * (W_up x)), silu(z) = z / (1 + e^-z),
 * fp32 accumulation, x as given (BF16), h in fp32.  MXFP4 launches of 2 to
 * 8 tokens with H and I multiples of 256 run on the scaled FP4 matrix
 * instruction, which takes its activations as e4m3: x enters as two e4m3
 * parts per element under a power-of-two scale per 32 (exact for a BF16
 * value unless it is 2^-15 or more below its block's largest) and h as
 * three (about 12 significant bits); products and sums stay fp32.  Only experts with a slot
 * contribute: y is the partial sum over the resident subset (the GPU side of
 * the pages' exact split); non-resident pairs are skipped.
 * One persistent kernel per launch of up to moe_decode_launch_tokens(desc)
 * tokens (a larger T is split evenly into launches in stream order).  The
 * gate/up rows of all selected experts are split evenly over the grid (on
 * the matrix core in whole multiples of 8 groups of 8 rows), h is handed
 * between workgroups through the workspace tagged with the launch's
 * generation, then the down rows are split over the grid (evenly, or on the
 * matrix core by cost: an expert's rows weigh more the more tokens chose
 * it) and each row's gate-weighted result is added into y with an fp32
 * atomic, so the summation order (and the last bits of y) can differ
 * between runs.
 *   x              device [T][H] BF16;   1 <= T <= MOE_DECODE_MAX_T
 *   ids, w         device [T][k] (from moe_route or the caller)
 *   slot_of_expert device [E] int32: slot holding expert e, -1 = not
 *                  resident; NULL = identity (expert e in slot e)
 *   slot_pool      device base; slot s starts at slot_pool + s * bytes
 *                  (bytes from moe_expert_layout, 256-byte aligned)
 *   shared_expert  device block in the same layout, or NULL (required iff
 *                  desc->has_shared)
 *   y              device out [T][H] float, overwritten
 *   ws             device workspace, moe_workspace_bytes(.., MOE_MODE_DECODE)
 * ids outside [0, E) are an error the kernels cannot report: they are
 * skipped.
 * Co-residency: the grid is sized so that all its workgroups fit the device
 * at once (at most two per compute unit, capped by occupancy), because
 * workgroups wait for each other's logits, h and cleared y.  Every such wait
 * is bounded: if other work keeps compute units busy past the bound (an
 * oversubscribed device), the wait gives up, y is wrong, and the workspace's
 * wait-expired word is set; moe_decode_status reads and clears it. */
int moe_decode(const moe_desc* desc, const void* x, int32_t T,
               const int32_t* ids, const float* w,
               const int32_t* slot_of_expert, const void* slot_pool,
               const void* shared_expert, float* y, void* ws, size_t ws_bytes,
               void* stream);

/* moe_route_decode: moe_route followed by moe_decode as one call: the
 * router's dot products, softmax and top-k run inside the same persistent
 * kernel as the experts (every workgroup takes a share of the router rows,
 * hands its logits to all others through the workspace, and ranks the tokens
 * itself), so one launch per batch of up to 16 tokens does the whole layer.
 * The router's ids and w are written out as by moe_route (the host side of a
 * miss split needs them) and y as by moe_decode.  Same arguments as
 * moe_decode plus w_router (device, [E][H] in desc->router_wtype); ids and w
 * are outputs.  ws: moe_workspace_bytes(.., MOE_MODE_DECODE).  The
 * co-residency note and the wait-expired word of moe_decode apply. */
int moe_route_decode(const moe_desc* desc, const void* x, const void* w_router,
                     int32_t T, int32_t* ids, float* w,
                     const int32_t* slot_of_expert, const void* slot_pool,
                     const void* shared_expert, float* y, void* ws,
                     size_t ws_bytes, void* stream);

/* moe_decode_launch_tokens: tokens one decode kernel launch takes for this
 * layer shape (at most 16; fewer when the LDS stages of x, or of h on the
 * matrix-core MXFP4 path, would not fit); moe_decode and moe_route_decode
 * split a larger T evenly into ceil(T / this) launches.  Host only.  A
 * negative MOE_E* code if the shape has no decode kernel. */
int32_t moe_decode_launch_tokens(const moe_desc* desc);

/* moe_decode_status: the decode workspace's wait-expired word (non-zero when
 * a bounded wait inside a moe_decode / moe_route_decode launch on this
 * workspace gave up, so that launch's y is wrong) is copied to *status
 * (device int32; NULL = do not copy), then cleared when `clear` is non-zero.
 * Enqueued on `stream` after the calls it should cover; read *status after
 * synchronising.  The word is sticky: it stays set across calls until
 * cleared, so one query after a run of calls covers all of them.
 * MOE_EWORKSPACE if ws is not a decode workspace (< 8 KB or unaligned). */
int moe_decode_status(void* ws, size_t ws_bytes, int32_t* status, int32_t clear, void* stream);

/* moe_route_decode_noalloc: moe_route_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments and results as
 * moe_route_decode, without a workspace: the decode workspace is a
 * file-scope device array of MOE_NOALLOC_SCRATCH_BYTES that each GPU holds
 * until the process ends (its address is looked up once per device; the
 * first call on a device clears it with a kernel on `stream`).  A batch
 * whose moe_workspace_bytes(.., T, MOE_MODE_DECODE) exceeds the array is
 * rejected with MOE_EWORKSPACE.  No call allocates or frees anything.  Every
 * call on one GPU shares its array: calls that can overlap on one GPU (other
 * streams, other host threads) race.  wait_status: device int32 that
 * receives the wait-expired word of this call's launches (0 = every wait
 * finished in time; see moe_decode_status), or NULL. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_route_decode_noalloc(const moe_desc* desc, const void* x, const void* w_router,
                             int32_t T, int32_t* ids, float* w,
                             const int32_t* slot_of_expert, const void* slot_pool,
                             const void* shared_expert, float* y, int32_t* wait_status,
                             void* stream);

/* moe_prefill: the same layer for long token batches.  Pairs are
 * counting-sorted by expert and each expert's rows run as a grouped GEMM.
 * MXFP4 weights: x and h are quantised to MXFP4 on the fly (x along H, h
 * along I, same encoder as moe_quantize_mxfp4) and both expert products run
 * on the scaled FP4 matrix cores with fp32 accumulation.  NVFP4 weights:
 * each weight is expanded to e2m1 x E4M3 in BF16 (exact) and both products
 * run on the BF16 matrix cores with x as given and h rounded to BF16, the
 * fp32 matrix scales applied to the fp32 results.  The down product writes
 * each pair's output to the workspace and a last step sums a token's pairs
 * in rank order times their gate weights (the shared expert last, weight 1):
 * the result does not depend on scheduling.  Prefill routes nearly every
 * expert (explainx.ai guide, "Prefill: load almost every expert without
 * idling the GPU").  Arguments as moe_decode; 1 <= T <= 65536; hidden and
 * inter multiples of 128; ws of moe_workspace_bytes(.., PREFILL). */
int moe_prefill(const moe_desc* desc, const void* x, int32_t T,
                const int32_t* ids, const float* w,
                const int32_t* slot_of_expert, const void* slot_pool,
                const void* shared_expert, float* y, void* ws, size_t ws_bytes,
                void* stream);

/* moe_debug_prefill_layout: where a prefill workspace for T tokens keeps the
 * expert sort, for tests of the sort's integers: out[0] byte offset of
 * seg_start (int32 [E + 2]: first sorted position of each bin, bins 0..E-1
 * the routed experts, bin E the shared expert, then the total), out[1] of
 * the tile list (int32: the count, then (bin, first sorted position) per
 * 128-row tile in bin order), out[2] of sorted_pair (int32: pair ids t*k + j,
 * or T*k + t for the shared expert, stably sorted by bin; non-resident pairs
 * left out), out[3] the tile list's capacity, out[4] the number of pairs. */
int moe_debug_prefill_layout(const moe_desc* desc, int32_t T, int64_t out[5]);

/* moe_merge_partials: y = a + b elementwise over n floats (device).  The
 * exact merge of two partial sums computed over disjoint expert subsets
 * (explainx.ai guide, "Decode: ..."; ainewsfeed.tech article, third
 * paragraph).  y may alias a or b. */
int moe_merge_partials(const float* a, const float* b, float* y, size_t n,
                       void* stream);

/* ---- formats ----------------------------------------------------------- */
/* moe_quantize_mxfp4: src [rows][K] float (row stride src_ld floats) ->
 * codes [rows][K/2], scales [rows][K/32] (device).  Per 32-block: a = max|v|;
 * a == 0 -> scale 0, codes 0; else X = floor(log2 a) - 2 clamped to
 * [-127, 127], scale byte X + 127, codes = v / 2^X rounded to e2m1 with
 * round-to-nearest-even, saturating at 6, sign kept.  K % 32 == 0. */
int moe_quantize_mxfp4(const float* src, int32_t rows, int32_t K,
                       int64_t src_ld, uint8_t* codes, uint8_t* scales,
                       void* stream);

/* moe_pack_expert: write one expert into its block (dst, device, 256-byte
 * aligned, moe_expert_layout bytes) from gate [I][H], up [I][H], down [H][I]
 * (device, row-major, src_type MOE_WTYPE_F32 or MOE_WTYPE_BF16).  BF16
 * experts: values rounded to BF16 (nearest even) if given as fp32.  MXFP4
 * experts: quantised with the encoder of moe_quantize_mxfp4 (blocks along
 * K = H for gate/up, K = I for down).  Host and device blocks share this
 * layout, so the same bytes serve the pinned pool and the slots. */
int moe_pack_expert(const moe_desc* desc, const void* gate, const void* up,
                    const void* down, int32_t src_type, void* dst, void* stream);

/* moe_debug_dequant_mxfp4: n_blocks MXFP4 blocks (codes 16 B each, one scale
 * byte each) -> 32 * n_blocks floats, value e2m1(code) * 2^(s-127) computed
 * by the fp32 in-register convert the decode kernels' down rows use (the
 * gate/up rows' BF16 convert is checked through moe_debug_dot_fp4).  Test
 * hook. */
int moe_debug_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales,
                            int64_t n_blocks, float* out, void* stream);

/* moe_debug_dot_fp4: for every block b < n_blocks and x vector v < n_x,
 * out[b * n_x + v] = the per-block step of the decode kernels' gate/up rows
 * on block b and 32 BF16 values x[v][0..32): MXFP4 (wtype MOE_WTYPE_MXFP4):
 * the 32 e2m1 codes converted to BF16 by the same in-register convert, dotted
 * with x in fp32, times the block's e8m0 scale (scales[b]); NVFP4
 * (MOE_WTYPE_NVFP4): the sums over the two 16-element halves, each times its
 * E4M3 scale (scales[2b], scales[2b+1]), the matrix scale not applied.
 * codes [n_blocks][16] bytes, x [n_x][32] BF16, all device.  With x a
 * one-hot vector the result is one element's exact value.  Test hook. */
int moe_debug_dot_fp4(int32_t wtype, const uint8_t* codes, const uint8_t* scales,
                      const void* x, int64_t n_blocks, int32_t n_x, float* out, void* stream);

/* moe_debug_mfma_fp4_tile: D = A . B^T for one 16 x 128 MXFP4 tile of A
 * (a_codes [16][64] bytes, a_scales [16][4]) and of B (same shapes), out
 * [16][16] float row-major, computed by one wave through the fragment
 * loaders and scaled FP4 matrix instruction that moe_prefill uses.  Test
 * hook for the operand and result lane layouts. */
int moe_debug_mfma_fp4_tile(const uint8_t* a_codes, const uint8_t* a_scales,
                            const uint8_t* b_codes, const uint8_t* b_scales,
                            float* out, void* stream);

/* moe_debug_wave_scan: out[64 w + l] = in[64 w] + ... + in[64 w + l] for
 * w < n_waves, l < 64 (int32, device buffers of 64 n_waves), through the DPP
 * wave scan the decode kernel builds its expert list with (test hook). */
int moe_debug_wave_scan(const int32_t* in, int32_t* out, int32_t n_waves, void* stream);

/* moe_debug_read_probe: read `bytes` (multiple of 16) of device memory with
 * 16-byte loads from `blocks` workgroups of 256 threads, 8 loads in flight
 * per thread; writes nothing unless a checksum hits a magic value.  Timed by
 * the caller to measure the attainable HBM read rate the roofline fractions
 * can be compared with. */
int moe_debug_read_probe(const void* buf, size_t bytes, int32_t blocks,
                         uint32_t* out, void* stream);

/* ---- q* split ---------------------------------------------------------- */
/* Number of the m cache misses to fill into GPU slots so that the PCIe fills
 * (rate b_pcie) and host-side execution of the rest (rate b_host) finish
 * together: argmin over q in [0, m] of max(q / b_pcie, (m - q) / b_host),
 * ties to the larger q.  The pages name this policy q* and say it is chosen
 * from profiled bandwidths so that neither path idles (futuresignalnews.com,
 * "1. Bandwidth-Adaptive Execution (The q* Policy)"; explainx.ai, "Decode:
 * ..."); the formula is the reading used.  Returns -1 for m < 0 or
 * non-positive rates. */
int32_t moe_qstar(int32_t m, double b_pcie, double b_host);

/* ---- global LRU planner (host only, no HIP calls) ---------------------- */
/* A global LRU over (layer, expert) keys and n_slots numbered slots: one
 * cache shared by every layer, following the router ("FreeToken 753b Model
 * Explained", "How MoE Paging and Caching Work").  Per plan call (one layer,
 * one step): the step's selected set S is the distinct ids in
 * first-appearance order; hits refresh recency in S order; misses are ranked
 * by summed gate weight (descending, ties to the lower id); the first q are
 * filled, each into the lowest empty slot, else the least recently used slot
 * whose key is not in S; unfilled misses stay out of the cache.  q is
 * clamped to [0, min(misses, n_slots - hits)]; q < 0 means q* from the
 * planner's bandwidths (moe_planner_set_bandwidths). */
#define MOE_PLAN_MAX 256
typedef struct moe_plan {
  int32_t layer;
  int32_t n_selected;                    /* |S|                              */
  int32_t n_hits, n_misses;
  int32_t q;                             /* fills actually planned           */
  int32_t n_host;                        /* misses left to the host side     */
  int32_t selected[MOE_PLAN_MAX];        /* S, first-appearance order        */
  int32_t hits[MOE_PLAN_MAX];            /* S order                          */
  int32_t misses[MOE_PLAN_MAX];          /* S order                          */
  int32_t fill_expert[MOE_PLAN_MAX];     /* ranked order, q entries          */
  int32_t fill_slot[MOE_PLAN_MAX];
  int32_t victim_layer[MOE_PLAN_MAX];    /* -1 when the slot was empty       */
  int32_t victim_expert[MOE_PLAN_MAX];
  int32_t host_expert[MOE_PLAN_MAX];     /* ranked order, n_host entries     */
  int32_t hit_slot[MOE_PLAN_MAX];        /* slot of each hit                 */
} moe_plan;

typedef struct moe_planner moe_planner;
/* n_layers, n_experts >= 1; 1 <= n_slots. The cache starts cold. */
int moe_planner_create(moe_planner** out, int32_t n_layers, int32_t n_experts,
                       int32_t n_slots);
void moe_planner_destroy(moe_planner* p);
int moe_planner_set_bandwidths(moe_planner* p, double b_pcie, double b_host);
/* ids/w: host, n entries (a step's T*k pairs); at most MOE_PLAN_MAX distinct
 * ids (else MOE_ECACHE); ids outside [0, n_experts) -> MOE_EINVAL.  On error
 * the planner state is unchanged. */
int moe_planner_plan(moe_planner* p, int32_t layer, const int32_t* ids,
                     const float* w, int32_t n, int32_t q, moe_plan* plan);
/* Undo the last successful moe_planner_plan (one level). */
int moe_planner_rollback(moe_planner* p);
/* slot of each expert of `layer` (-1 = not resident), host out [n_experts] */
int moe_planner_slot_table(const moe_planner* p, int32_t layer, int32_t* out);
/* Rebuild the cache state under a budget of n_slots (>= 1) slots: the
 * n_slots most recently used residents survive (ties to the lower slot) and
 * keep their recency; a survivor whose slot is below n_slots stays there,
 * the others move, in old-slot order, into the free slots below n_slots in
 * ascending order; the rest are evicted.  old_of_new: host out [n_slots],
 * the old slot each new slot's expert comes from (-1 = empty).  The pages
 * rebuild the GPU expert cache under a revised VRAM budget at scheduler safe
 * points without restarting or reloading the host pool (futuresignalnews.com,
 * "3. Elastic Memory Management"); which experts survive and where they go is
 * the reading used.  Drops the rollback level. */
int moe_planner_resize(moe_planner* p, int32_t n_slots, int32_t* old_of_new);
int32_t moe_planner_n_slots(const moe_planner* p);

/* ---- expert cache: planner + async fills from a pinned host pool ------- */
/* moe_cache_create keeps the caller's pointers until moe_cache_destroy:
 *   host_pool          pinned host memory, [n_layers][n_experts] blocks of
 *                      expert_bytes (hipHostMalloc / torch pin_memory)
 *   dev_slot_pool      device, n_slots blocks of expert_bytes
 *   dev_slot_of_expert device [n_layers][n_experts] int32, set to -1 here
 *                      (on the null stream) and kept equal to the planner's
 *                      table by cache_fill (ordered on the compute stream)
 * It creates HIP events (one per slot plus one per fill batch). */
typedef struct moe_cache moe_cache;
int moe_cache_create(moe_cache** out, const void* host_pool, int32_t n_layers,
                     int32_t n_experts, size_t expert_bytes,
                     void* dev_slot_pool, int32_t n_slots,
                     int32_t* dev_slot_of_expert);
void moe_cache_destroy(moe_cache* c);
int moe_cache_set_bandwidths(moe_cache* c, double b_pcie, double b_host);
/* Plan one step of one layer (see the planner above). */
int moe_cache_plan(moe_cache* c, int32_t layer, const int32_t* ids_host,
                   const float* w_host, int32_t n, int32_t q, moe_plan* plan);
/* cache_fill: for each planned fill, side_stream waits until the victim
 * slot's last use (recorded by moe_cache_release) has finished, then one
 * hipMemcpyAsync copies the expert's block from the pinned host pool into its
 * slot; compute_stream then waits for the copies and the device slot table
 * is updated on compute_stream (victims -> -1, fills -> slot).  Returns
 * without waiting.  Miss option "copy over PCIe, run on the GPU, keep
 * cached" (explainx.ai guide, "Decode: ...").  On failure the planner is
 * rolled back, slots whose copy may have started are marked empty, and
 * MOE_EHIP / MOE_ECACHE is returned. */
int cache_fill(moe_cache* c, const moe_plan* plan, void* side_stream,
               void* compute_stream);
/* Record, on compute_stream, the last use of every slot the plan reads
 * (hits and fills); call after the step's moe_decode is enqueued. */
int moe_cache_release(moe_cache* c, const moe_plan* plan, void* compute_stream);
/* Rebuild the cache under a new budget of n_slots at a safe point (between
 * steps: after the last step's moe_cache_release): moe_planner_resize's rule,
 * then, on compute_stream, one device-to-device copy per survivor that
 * changes address and the device slot table updated (evicted -> -1, moved ->
 * new slot).  dev_slot_pool (caller-owned, n_slots blocks of expert_bytes)
 * is either the current pool (shrinking in place: no copy overlaps) or a
 * range disjoint from it (else MOE_EINVAL); the old pool must stay allocated
 * until compute_stream has passed this call.  Fills after the rebuild wait
 * for it.  Elastic memory management (futuresignalnews.com, "3. Elastic
 * Memory Management"; "FreeToken 753b Model Explained", "How MoE Paging and
 * Caching Work"). */
int moe_cache_resize(moe_cache* c, void* dev_slot_pool, int32_t n_slots,
                     void* compute_stream);
/* Test hook: make the next n cache_fill calls fail before any copy. */
int moe_cache_debug_fail_fills(moe_cache* c, int32_t n);
const moe_planner* moe_cache_planner(const moe_cache* c);

/* ---- full-layer prefill streaming -------------------------------------- */
/* A long prompt routes to nearly every expert of a layer, so prefill streams
 * whole layers from the pinned host pool; with two full-layer buffers the
 * next layer is copied over PCIe while the GPU computes the current one
 * (explainx.ai guide, "Prefill: load almost every expert without idling
 * the GPU"; futuresignalnews.com article, "2. Semantic-Aware Caching").  One buffer gives the pages' ablation (copy, then compute).
 *   host_pool  pinned host memory, [n_layers] blocks of layer_bytes (a
 *              layer's expert blocks in slot order, e.g. its E routed experts
 *              then its shared expert)
 *   dev_buf0/1 caller-owned device buffers of layer_bytes each; dev_buf1 NULL
 *              = single buffer.  Kept until moe_layer_stream_destroy.
 * Creates HIP events; the object is single-threaded. */
typedef struct moe_layer_stream moe_layer_stream;
int moe_layer_stream_create(moe_layer_stream** out, const void* host_pool,
                            int32_t n_layers, size_t layer_bytes, void* dev_buf0,
                            void* dev_buf1);
void moe_layer_stream_destroy(moe_layer_stream* s);
/* Make `layer` resident for the work enqueued next on compute_stream: if its
 * buffer (layer mod buffers) does not hold it yet, one hipMemcpyAsync on
 * copy_stream after the buffer's last release; compute_stream then waits for
 * the copy.  With two buffers the copy of layer + 1 is issued at once into
 * the other buffer if that buffer's layer has been released.  *dev_layer =
 * the device block of the layer.  MOE_ECACHE if the buffer still holds an
 * unreleased layer. */
int moe_layer_stream_acquire(moe_layer_stream* s, int32_t layer, void* copy_stream,
                             void* compute_stream, void** dev_layer);
/* The layer's work is enqueued on compute_stream: its buffer may be
 * refilled after that work. */
int moe_layer_stream_release(moe_layer_stream* s, int32_t layer, void* compute_stream);

/* ---- bandwidth probe --------------------------------------------------- */
/* Measures pinned host->device copy bandwidth (bytes / s) from `pinned_host`
 * into `dev` (both >= bytes) on `stream`, and host-memory streaming read
 * bandwidth over `pinned_host` with `threads` CPU threads (0 = all), best of
 * `reps`.  Blocks the caller.  The pages profile exactly these two rates
 * before splitting misses ("FreeToken 753b Model Explained", "Measure System
 * Bandwidth"). */
int moe_probe_bandwidths(const void* pinned_host, void* dev, size_t bytes,
                         int32_t reps, int32_t threads, void* stream,
                         double* b_pcie, double* b_host);

/* ---- host side of the split -------------------------------------------- */
/* moe_host_experts: the expert FFNs of the pairs left to the host, on the
 * host cores, reading expert blocks straight from a (pinned) host pool:
 *   y[t] = sum over pairs (t, j) with include[t*k + j] != 0 of
 *          w[t][j] * FFN_{ids[t][j]}(x[t])
 * with the moe_decode precision contract (x BF16 as given, fp32
 * accumulation, h in fp32).  A miss can stay where it lives and run there,
 * its partial sum merged exactly with the GPU's (explainx.ai guide,
 * "Decode: decide whether to move an expert or compute where it lives").
 *   x          host [T][H] BF16
 *   ids, w     host [T][k]
 *   include    host [T][k] bytes, non-zero = computed here; NULL = all pairs
 *   host_pool  host blocks of expert_bytes in the moe_expert_layout format
 *   host_index host [E]: block index of each expert in host_pool; NULL =
 *              block e holds expert e.  An included expert without a block
 *              (index < 0) is MOE_EINVAL.
 *   y          host [T][H] float, overwritten
 *   n_threads  host threads (0 = all hardware threads); a persistent pool
 *              is kept between calls.  Calls from several host threads are
 *              safe: they take the pool one after another.
 * Weights: BF16, MXFP4 or NVFP4 blocks.  Blocks the caller.  The shared
 * expert is not part of this call. */
int moe_host_experts(const moe_desc* desc, const void* x, int32_t T,
                     const int32_t* ids, const float* w, const uint8_t* include,
                     const void* host_pool, const int32_t* host_index,
                     float* y, int32_t n_threads);

/* moe_host_expert_rate: expert bytes per second moe_host_experts streams
 * from host_pool on one token over its first n_experts_timed experts, best of
 * reps: the host expert-kernel rate the q* split uses as b_host (the pages
 * profile the host side's own rate, "FreeToken 753b Model Explained",
 * "Measure System Bandwidth"). */
int moe_host_expert_rate(const moe_desc* desc, const void* host_pool,
                         int32_t n_experts_timed, int32_t reps, int32_t n_threads,
                         double* bytes_per_s);

/* ---- misc -------------------------------------------------------------- */
const char* moe_last_error(void);
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
