/*
 * ds4moe -- routed 2-bit mixture-of-experts FFN layer for AMD MI355X (gfx950).
 *
 * One layer of a DeepSeek-V4-Flash-style model whose routed experts are stored
 * in asymmetric 2-bit super-blocks while the router and the shared expert stay
 * at higher precision (ds4 README, "Models" section, as translated on
 * molayo1419.me: only the routed MoE experts are quantized; routing, shared
 * experts and projections are left alone).  The same layer also runs on
 * routed experts with 4-bit codes in the same super-block (the higher-quality
 * weight option the README lists beside the 2-bit one).  Per token t the
 * layer computes
 *
 *   l[t,e] = fp32( sum_h x[t,h] * Wr[e,h] + b[e] )      (fp64 accumulation)
 *   s      = sqrt(softplus(l)), softplus evaluated in the stable form
 *            max(l,0) + log1p(exp(-|l|)), log1p(u) by the series
 *            u - u^2/2 + u^3/3 - u^4/4 when u < 1/32 (opensource-hub.com
 *            "antirez/ds4" page, FAQ #1, router numeric test)
 *   top-k experts by logit, ties to the lower index; w_j = s_j / sum_i s_i
 *   h_j    = silu(Wg_e x_t) * (Wu_e x_t)                (dequant-fused)
 *   y[t]   = sum_j w_j * (Wd_e h_j)  [+ shared expert FFN(x_t), bf16 weights]
 *
 * CONVENTIONS (all entry points)
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns
 *     every buffer; the library never allocates, frees or keeps a pointer
 *     after a call returns.  Scratch memory comes from the caller's workspace,
 *     sized by ds4moe_workspace_bytes() (one exception:
 *     ds4moe_forward_decode_noalloc, whose scratch is a fixed array per GPU).
 *   - Calls only enqueue work on `stream` (a hipStream_t passed as void*,
 *     NULL = the null stream) and return; there is no host synchronisation.
 *   - The small descriptor structs are HOST memory, read during the call only.
 *   - Every argument is validated on the host before anything is launched; a
 *     non-zero ds4moe_status is returned and nothing is enqueued.  A HIP launch
 *     failure returns DS4MOE_ERR_HIP.  No exceptions cross this boundary.
 *   - Device pointers must be 16-byte aligned.
 *   - Same inputs, same stream order => bitwise identical outputs (no
 *     floating-point atomics anywhere).
 *   - Calls that share a workspace must not overlap.
 */
#ifndef DS4MOE_H
#define DS4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DS4MOE_OK = 0,
  DS4MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  DS4MOE_ERR_SHAPE = 2,       /* a size is out of the supported range */
  DS4MOE_ERR_DTYPE = 3,       /* unknown dtype code */
  DS4MOE_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
  DS4MOE_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  DS4MOE_ERR_UNSUPPORTED = 6, /* valid request this build does not implement */
  DS4MOE_ERR_HIP = 7,         /* a HIP launch or runtime call failed */
  DS4MOE_ERR_HOSTMEM = 8      /* host expert weights are not pinned (device-visible) host memory */
} ds4moe_status;

typedef enum { DS4MOE_F32 = 0, DS4MOE_BF16 = 1 } ds4moe_dtype;

typedef enum { DS4MOE_MODE_ROUTE = 0, DS4MOE_MODE_DECODE = 1, DS4MOE_MODE_PREFILL = 2 } ds4moe_mode;

/* Layer shape (host struct).
 *   hidden        H: multiple of 256, 256..65536
 *   inter         I: routed expert intermediate; multiple of 16 and either a
 *                 multiple of 256 or a divisor of 256
 *   n_experts     E: top_k <= E <= 256
 *   top_k         k: 1..16
 *   shared_inter  Is: 0 (no shared expert) or a multiple of 32
 *   x_dtype       dtype of x: DS4MOE_F32 or DS4MOE_BF16.  The expert
 *                 products take fp16 operands: each token enters them as
 *                 x * 2^-e with max |x| in [2^e, 2^(e+1)), and its SwiGLU
 *                 intermediate as h * 2^-2e, so activations of any finite
 *                 magnitude (the whole bf16 / fp32 range) are represented
 *                 to fp16 precision relative to the token's largest element
 *                 and the result carries 2^2e back exactly (results are
 *                 finite while y itself fits fp32)
 *   router_dtype  dtype of Wr: DS4MOE_F32 or DS4MOE_BF16
 *   expert_bits   code width of the packed routed experts: 2, 4, 5 or 6
 *                 (gate and up, and down unless down_bits says otherwise;
 *                 5-bit codes are packed into 6-bit units, see ds4moe_pack)
 *   down_bits     code width of the routed down matrices: 0 (= expert_bits),
 *                 2, 4, 5 or 6.  The pages' quant mixes give the down projection a
 *                 format of its own (molayo1419.me "antirez-ds4" insight,
 *                 "Models" section: ds4's 2-bit model stores routed gate/up
 *                 and routed down in different block types; the GLM notes
 *                 pair 2- to 5-bit gate/up with down up to 6 bits) */
typedef struct {
  int32_t hidden;
  int32_t inter;
  int32_t n_experts;
  int32_t top_k;
  int32_t shared_inter;
  int32_t x_dtype;
  int32_t router_dtype;
  int32_t expert_bits;
  int32_t down_bits;
} ds4moe_dims;

/* Weights (host struct of device pointers).
 *   router_w   [E,H] row-major, router_dtype
 *   router_bias [E] fp32, or NULL: added to the logit, so it moves both the
 *              selection and the weights
 *   gate, up   E packed matrices W[I,H] each (ds4moe_pack layout with
 *              dims->expert_bits), expert e at byte offset
 *              e * ds4moe_packed_bytes_bits(I, H, expert_bits)
 *   down       E packed matrices W[H,I] (width down_bits, or expert_bits
 *              when down_bits is 0), expert e at
 *              e * ds4moe_packed_bytes_bits(H, I, that width)
 *   sh_gate, sh_up  [Is,H] bf16 row-major; sh_down [H,Is] bf16; all NULL
 *              when shared_inter == 0.  The shared expert is computed with
 *              fp16 operands: its weights must lie inside the binary16 range. */
typedef struct {
  const void *router_w;
  const float *router_bias;
  const void *gate;
  const void *up;
  const void *down;
  const void *sh_gate;
  const void *sh_up;
  const void *sh_down;
} ds4moe_weights;

/* Optional routing outputs (host struct of device pointers; each may be NULL).
 *   topk_idx [T,k] int32  selected experts in rank order (logit descending,
 *                         ties to the lower expert index)
 *   topk_w   [T,k] fp32   normalised weights, sum over j = 1
 *   counts   [E]   int32  assignments per expert
 *   offsets  [E+1] int32  exclusive prefix sum of counts, offsets[E] = T*k
 *   perm     [T*k] int32  assignment ids a = t*k + j grouped by expert, in
 *                         increasing t within an expert
 *   logits   [T,E] fp32   router logits */
typedef struct {
  int32_t *topk_idx;
  float *topk_w;
  int32_t *counts;
  int32_t *offsets;
  int32_t *perm;
  float *logits;
} ds4moe_routing;

/* Bytes of one packed matrix of `rows` x `cols` weights (cols = reduction
 * length) with `bits`-bit codes (2, 4, 5 or 6).  Same byte count as the
 * canonical blocks (84 bytes per 256 weights, 2.625 bits per weight, with
 * 2-bit codes; 148 bytes, 4.625 bits per weight, with 4-bit codes; 212
 * bytes, 6.625 bits per weight, with 6-bit codes) when cols is a multiple of
 * 256; 5-bit codes are packed into the 6-bit unit (212 bytes per 256
 * weights, against 180 canonical).  A divisor of 256 is padded to 256.
 * Returns 0 for an unsupported shape or width (rows, cols above 2^31
 * included). */
size_t ds4moe_packed_bytes_bits(int64_t rows, int64_t cols, int32_t bits);

/* ds4moe_packed_bytes_bits(rows, cols, 2). */
size_t ds4moe_packed_bytes(int64_t rows, int64_t cols);

/* Repack canonical super-blocks into the HBM layout the GEMV/GEMM kernels
 * stream (the canonical block is the 2-bit K-quant super-block named in the
 * ds4 README "Models" section: 256 weights = 16 sub-blocks of 16, 4-bit
 * scale (low nibble) and 4-bit min (high nibble) per sub-block, 2-bit codes
 * four per byte lowest bits first, fp16 d and dmin; w = d*scale*q - dmin*min).
 *   dst        packed output, n_mats * ds4moe_packed_bytes(rows, cols) bytes
 *   canonical  n_mats matrices of rows*cols/256 blocks of 84 bytes each:
 *              scales[16] @0, qs[64] @16, d @80, dmin @82 (little-endian);
 *              blocks tile the row-major flattened matrix
 *   rows       multiple of 16;  cols  multiple of 16, and a multiple of 256
 *              or a divisor of 256
 * Packed layout: units of 16 rows x 256 columns, 1344 bytes each, unit
 * (row_tile, col_chunk) at ((row_tile * nchunks) + col_chunk) * 1344:
 *   [0,1024)    2-bit codes, 16 bytes per MFMA lane (lane = 16*g + r, row r);
 *               dword u of lane (r,g) holds sub-block 4u+g of row r, element
 *               i at bits 4*(i%8) + 2*(i/8)
 *   [1024,1280) per row 16 bytes: bytes 2g and 2g+1 (g < 4) hold the scales
 *               of sub-blocks g | 8+g<<4 and 4+g | 12+g<<4; bytes 8-11 and
 *               12-15 hold the mins of sub-blocks 0-7 and 8-15, byte b of each
 *               group holding sub-block b (low nibble) and b+4 (high nibble)
 *   [1280,1344) per row d (bits 0-15) and dmin (bits 16-31), binary16
 * The conversion is exact: no value is altered.  Same as ds4moe_pack with
 * bits = 2. */
int ds4moe_pack_q2k(void *dst, const void *canonical, int64_t n_mats, int64_t rows, int64_t cols, void *stream);

/* Repack canonical super-blocks with `bits`-bit codes (2, 4, 5 or 6).
 * bits = 2: the blocks and units of ds4moe_pack_q2k.
 * bits = 4: canonical blocks of 148 bytes: scales[16] @0 as above, qs[128]
 *   @16 (weight i at byte i/2, bits 4*(i%2)), d @144, dmin @146; w =
 *   d*scale*q - dmin*min with q in 0..15.  Units of 16 rows x 256 columns,
 *   2368 bytes each, at ((row_tile * nchunks) + col_chunk) * 2368:
 *   [0,2048)    two code planes of 1024 bytes, 16 bytes per MFMA lane
 *               (lane = 16*g + r, row r) in each: dword 4p+v of lane (r,g)
 *               lies in plane p at 16*lane + 4*v; dword 2u+h holds elements
 *               8h..8h+7 of sub-block 4u+g of row r, element 8h+e in the
 *               nibble 2e (e < 4) or 2(e-4)+1 (e >= 4)
 *   [2048,2304) scales and mins per row, as in the 2-bit unit
 *   [2304,2368) per row d | dmin<<16, as in the 2-bit unit
 * bits = 5 or 6: canonical blocks of 180 or 212 bytes: scales[16] @0 as
 *   above, the 256 codes as one bit stream from byte 16, lowest bits first
 *   (weight i at bits b*i .. b*i+b-1: the order of the 2- and 4-bit blocks),
 *   d and dmin after them; q in 0..2^b-1 (the pages' GLM notes pair 5-bit
 *   gate/up with down up to 6 bits: molayo1419.me ds4 README translation,
 *   "Models" section).  Units of 16 rows x 256 columns, 3392 bytes each:
 *   [0,2048)    the low 4 bits of every code, laid out as the two planes of
 *               the 4-bit unit
 *   [2048,3072) the high 2 bits of every code, laid out as the plane of the
 *               2-bit unit (the top bit is zero for 5-bit codes)
 *   [3072,3328) scales and mins per row, as in the 2-bit unit
 *   [3328,3392) per row d | dmin<<16, as in the 2-bit unit
 * Arguments, alignment and status codes as ds4moe_pack_q2k; also
 * DS4MOE_ERR_SHAPE for a width other than 2, 4, 5 or 6, or 2^39 padded
 * weights or more in all.  Exact. */
int ds4moe_pack(void *dst, const void *canonical, int64_t n_mats, int64_t rows, int64_t cols, int32_t bits,
                void *stream);

/* Dequantize packed matrices to fp32, row-major [n_mats, rows, cols]:
 * w = d*scale*q - dmin*min, every product exact, one rounding (bitwise equal
 * to the correctly rounded value of the block's definition).  Same as
 * ds4moe_dequant with bits = 2. */
int ds4moe_dequant_q2k(float *dst, const void *packed, int64_t n_mats, int64_t rows, int64_t cols, void *stream);

/* ds4moe_dequant_q2k for units with `bits`-bit codes (2, 4, 5 or 6; 5 and 6
 * read the same unit); products of at most 21 significant bits, still one
 * rounding. */
int ds4moe_dequant(float *dst, const void *packed, int64_t n_mats, int64_t rows, int64_t cols, int32_t bits,
                   void *stream);

/* Workspace bytes needed by a call with `T` tokens in `mode`
 * (ds4moe_mode).  Never decreases with T within a mode, so a workspace sized
 * for the largest batch serves every smaller one.  Returns 0 if dims is NULL
 * or invalid. */
size_t ds4moe_workspace_bytes(const ds4moe_dims *dims, int32_t T, int32_t mode);

/* Router only: logits, scores, top-k, weights, per-expert histogram, scan and
 * stable permutation.  The router stays at high precision, as the routed
 * experts alone are quantized (molayo1419.me "antirez-ds4" insight, "Models"
 * section); the score is sqrt(softplus) in the stable form of the router
 * numeric test (opensource-hub.com "antirez/ds4" page, FAQ #1), where fp32
 * log(1 + exp(x)) loses its digits near logit -12.  x [T,H] in dims->x_dtype; T >= 0 (0 = no-op).
 * Needs router_w (and router_bias if any) in `w`; `out` (host struct) must
 * not be NULL but any field may be.  ws: ds4moe_workspace_bytes(dims, T, 0). */
int ds4moe_route(const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T,
                 ds4moe_routing *out, void *ws, size_t ws_bytes, void *stream);

/* Whole layer for a small batch, 1 <= T <= 16 (decode): every new token is
 * routed through the experts again, so decode streams the chosen experts'
 * 2-bit weights once per call (molayo1419.me "antirez-ds4" insight, SSD
 * streaming section: generation is the phase that re-reads routed experts;
 * the 16-token batch stands for the server's micro-batched sessions,
 * blog.123qwe.co.kr DwarfStar article, baseline table).  y [T,H] fp32 is
 * overwritten.  route_out (host struct, nullable) receives the routing.
 * ws: ds4moe_workspace_bytes(dims, T, DS4MOE_MODE_DECODE). */
int ds4moe_forward_decode(const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T, float *y,
                          ds4moe_routing *route_out, void *ws, size_t ws_bytes, void *stream);

/* Whole layer for any T >= 0 (prefill; T = 0 is a no-op): the tokens are
 * grouped by expert so that each expert's 2-bit weights are read once per
 * chunk and multiplied against all of its tokens (the 2048-token chunk of the
 * pages' prefill benchmark, blog.123qwe.co.kr DwarfStar article, "Repository
 * layout and evaluation" section).  Same arguments as
 * ds4moe_forward_decode; ws: ds4moe_workspace_bytes(dims, T, DS4MOE_MODE_PREFILL). */
int ds4moe_forward_prefill(const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T, float *y,
                           ds4moe_routing *route_out, void *ws, size_t ws_bytes, void *stream);

/* Kernel slots timed by ds4moe_forward_timed. */
#define DS4MOE_N_TIMED_KERNELS 11

/* For measurement: the same work as ds4moe_forward_decode (mode
 * DS4MOE_MODE_DECODE) or ds4moe_forward_prefill (DS4MOE_MODE_PREFILL); each
 * kernel is launched with a start/stop event pair that its own dispatch
 * stamps (hipExtLaunchKernelGGL), so event elapsed times are kernel
 * durations.  `events` is a host array of 2*DS4MOE_N_TIMED_KERNELS hipEvent_t
 * created by the caller; pair i = (events[2i], events[2i+1]) times slot i:
 * 0 router logits, 1 top-k (decode: top-k + permutation), 2 permutation
 * (prefill), 3 gate/up + SwiGLU, 4 down, 5 shared gate/up, 6 shared down,
 * 7 combine, 8 expert-cache plan, 9 expert-cache fill (those two only in
 * ds4moe_forward_decode_cached), 10 fp16 copy of the shared expert's bf16
 * weights (prefill with more than 64 tokens).  The events of a slot with no kernel in the
 * call are not recorded (they keep their last stamps), so a caller that
 * records its own event on the stream before the call tells those slots
 * apart: their start precedes it.  Any other mode returns DS4MOE_ERR_SHAPE; a
 * NULL array or event DS4MOE_ERR_NULL. */
int ds4moe_forward_timed(int32_t mode, const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T,
                         float *y, ds4moe_routing *route_out, void *ws, size_t ws_bytes, void *const *events,
                         void *stream);

/* MEASUREMENT: a plain streaming read, the ceiling the HBM-bound expert
 * kernels are compared against on the same GPU.  Reads `bytes` (a multiple
 * of 16) from the device buffer `buf` (16-byte aligned) with n_workgroups
 * (1..2^20) workgroups of 256 threads, each thread keeping 8 16-byte loads
 * in flight over a grid-stride loop, and writes one checksum word per
 * workgroup to sink[n_workgroups] (device, uint32).  start_event and
 * stop_event: both NULL, or two hipEvent_t created by the caller that the
 * kernel's own dispatch stamps (their elapsed time is the kernel duration).
 * Errors: DS4MOE_ERR_NULL, _SHAPE, _ALIGN before any launch; _HIP. */
int ds4moe_read_probe(const void *buf, size_t bytes, int32_t n_workgroups, uint32_t *sink, void *start_event,
                      void *stop_event, void *stream);

/* ROUTED-EXPERT CACHE.  The experts' packed matrices stay in
 * pinned host memory; a cache buffer in device memory holds n_slots expert
 * slots (gate, up and down of one expert each).  A call routes the batch,
 * gives every expert it uses a slot (a slot already holding the expert, else
 * the least recently used slot, ties to the lower slot index, never one the
 * batch uses), copies the missing experts from host memory into their slots
 * (the GPU reads the host memory directly), and runs the expert kernels on
 * the slots.  The outputs are bitwise those of ds4moe_forward_decode on the
 * same experts resident in device memory.  This is the bounded routed-expert
 * cache with loads on a miss of the pages' SSD streaming mode ("antirez-ds4"
 * insight page, SSD streaming section; DwarfStar architecture article,
 * "Memory trade-off: resident vs SSD streaming" section), with host memory
 * as the backing store; the pages fix no eviction policy.
 *
 * Bytes of the cache buffer for n_slots slots (1 <= n_slots <= E); 0 for
 * invalid dims or n_slots.  The pages size the cache as a byte budget or a
 * slot count, the automatic budget being 80 % of the working set without the
 * non-routed weights (aitrends.kr "antirez/ds4" trending page, SSD-streaming
 * bullet). */
size_t ds4moe_cache_bytes(const ds4moe_dims *dims, int32_t n_slots);

/* Empty every slot and zero the counters (one kernel on `stream`, no memset,
 * so it may be captured in a graph).  `cache` is a device buffer of at least
 * ds4moe_cache_bytes(dims, n_slots) bytes, 256-byte aligned, owned by the
 * caller.  Every later call on this buffer must pass the same dims and
 * n_slots.  Errors: DS4MOE_ERR_NULL, _ALIGN, _SHAPE (n_slots), _WORKSPACE
 * (cache_bytes too small). */
int ds4moe_cache_reset(const ds4moe_dims *dims, int32_t n_slots, void *cache, size_t cache_bytes, void *stream);

/* ds4moe_forward_decode (1 <= T <= 16) with the routed experts in host
 * memory: w->gate, w->up, w->down are HOST pointers into pinned memory
 * (hipHostMalloc, or a pinned torch tensor), in the same layout as the
 * device weights of ds4moe_forward_decode; router and shared-expert weights
 * are device pointers as there.  n_slots >= min(E, T*k) (every expert of the
 * batch holds a slot during the call).  events: NULL, or
 * 2*DS4MOE_N_TIMED_KERNELS events as for ds4moe_forward_timed.  Calls on one
 * cache buffer must not overlap (they update its state).  Errors: those of
 * ds4moe_forward_decode and ds4moe_cache_reset, and DS4MOE_ERR_HOSTMEM when
 * an expert pointer is not pinned host memory. */
int ds4moe_forward_decode_cached(const ds4moe_dims *dims, const ds4moe_weights *w, int32_t n_slots, void *cache,
                                 size_t cache_bytes, const void *x, int32_t T, float *y, ds4moe_routing *route_out,
                                 void *ws, size_t ws_bytes, void *const *events, void *stream);

/* ds4moe_forward_prefill (any T up to 2^20) with the routed experts in host
 * memory, as for ds4moe_forward_decode_cached (same weights convention, same
 * cache buffer, any 1 <= n_slots <= E).  A long batch may use more experts
 * than there are slots, so the used experts go through the slots in batches
 * of at most n_slots: the first batch holds every expert already cached (the
 * hits) and then misses in ascending expert order while slots remain, each
 * later batch the next n_slots misses; inside a batch each miss, in
 * ascending order, takes the least recently used slot (ties to the lower
 * slot index) that the batch has not taken, and a batch's misses are copied
 * in before its experts run.  Every used expert is copied at most once per
 * call, so a call copies max(0, used - cached) experts when the cache held
 * min(used, n_slots) of them.  The outputs are bitwise those of
 * ds4moe_forward_prefill on the same experts resident in device memory.
 * This is the pages' streaming mode serving long prefills, which it keeps
 * fast ("antirez-ds4" insight page, SSD streaming section; DwarfStar
 * architecture article, "Memory trade-off: resident vs SSD streaming"
 * section), with host memory as the backing store.  ws: ds4moe_workspace_bytes(dims, T,
 * DS4MOE_MODE_PREFILL).  Calls on one cache buffer must not overlap.
 * Errors: those of ds4moe_forward_prefill and ds4moe_cache_reset, and
 * DS4MOE_ERR_HOSTMEM when an expert pointer is not pinned host memory. */
int ds4moe_forward_prefill_cached(const ds4moe_dims *dims, const ds4moe_weights *w, int32_t n_slots, void *cache,
                                  size_t cache_bytes, const void *x, int32_t T, float *y, ds4moe_routing *route_out,
                                  void *ws, size_t ws_bytes, void *stream);

/* Enqueue a copy of the cache's counters since its reset to host memory
 * out[3] = {calls, hits, misses} (hits and misses count experts of calls);
 * read them after `stream` has synchronised. */
int ds4moe_cache_stats(const ds4moe_dims *dims, int32_t n_slots, const void *cache, size_t cache_bytes,
                       uint64_t *out, void *stream);

/* NO-ALLOCATION DECODE, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  ds4moe_forward_decode without a workspace argument: the
 * scratch memory is a fixed array of DS4MOE_NOALLOC_SCRATCH_BYTES in each
 * GPU's memory, held by the library from the first call on that GPU until
 * the process ends.  The call allocates nothing (no hipMalloc, no hipFree,
 * no allocating library routine); on a GPU's first call it looks up the
 * array's device address, with that GPU current on the calling thread.
 * Inputs, outputs and results are those of ds4moe_forward_decode (the same
 * kernels).  Shapes whose decode workspace (ds4moe_workspace_bytes(dims, T,
 * DS4MOE_MODE_DECODE)) exceeds the array return DS4MOE_ERR_WORKSPACE before
 * anything is launched; every other argument is checked as there, also
 * before any HIP call.  All calls on one GPU share its array: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  No state carries over from one call to the
 * next (the decode kernels read no scratch they did not write in the same
 * call), so nothing has to be cleared between calls. */
#define DS4MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

int ds4moe_forward_decode_noalloc(const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T,
                                  float *y, ds4moe_routing *route_out, void *stream);

/* Static description of a status code (never NULL). */
const char *ds4moe_status_str(int status);

/* Library ABI version (major*10000 + minor*100 + patch). */
int ds4moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DS4MOE_H */
