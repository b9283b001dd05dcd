// Routed-expert cache for small batches: every expert's packed matrices live
// in pinned host memory and a bounded set of S expert slots lives in device
// memory.  A call routes the batch, plans the slots of the experts it uses
// (least recently used slot on a miss), copies the missing experts from host
// memory into their slots, and runs the unchanged expert kernels on the slot
// arrays: the same bytes, so the same results as with resident experts.
//
// This is the bounded routed-expert cache with loads on a miss of the SSD
// streaming mode ("antirez-ds4" insight page, SSD streaming section; the
// DwarfStar architecture article, "Memory trade-off: resident vs SSD
// streaming" section), with host memory in the role of the disk and HBM in
// the role of RAM.  The pages fix no eviction policy; least recently used,
// ties to the lower slot, is the one taken here.
#include "common.h"
#include "launch.h"

namespace ds4 {

// Slots start empty (expert -1, stamp 0), counters at zero.
__global__ __launch_bounds__(256) void k_cache_reset(CacheState c, int S, int E) {
  if (threadIdx.x < sizeof(CacheHdr) / 4) reinterpret_cast<uint32_t *>(c.hdr)[threadIdx.x] = 0u;
  for (int s = threadIdx.x; s < S; s += 256) {
    c.slot_expert[s] = -1;
    c.stamp[s] = 0u;
  }
  for (int e = threadIdx.x; e < E; e += 256) c.expert_slot[e] = -1;
}

// The slot policy.  A call's used experts split into hits (already in a
// slot) and misses.  The misses, in ascending expert order, go through the
// slots in batches: batch 0 is the hits and the first S - hits misses, each
// later batch the next S misses (a small batch is batch 0 alone).  Batch j
// has stamp step+1+j; its hits take the stamp first, then each miss in
// order takes the slot with the smallest (stamp, slot) that the batch has
// not stamped, evicting its expert.  That sequence has a closed form:
//  * batch 0's misses take the slots that are not hits in (stamp, slot)
//    order, since every stamp before the call is below the batch's own;
//  * a later batch exists only when batch 0 filled every slot, and it
//    starts with every slot on the same stamp (the previous batch's), so its
//    i-th miss takes slot i.
// The plan kernels below compute it in parallel: one workgroup of 256
// threads (S <= E <= 256), thread t standing for slot t and for expert (or
// tile) t.

// Exclusive prefix sums, in thread order, of NV values per thread at once;
// tot[i] = the sum over the workgroup.  Ends with a barrier.
template <int NV>
__device__ __forceinline__ void block_scan(int (&v)[NV], int (&tot)[NV], int (*lds)[4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) x[i] = v[i];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int y = __shfl_up(x[i], o);
      if (lane >= o) x[i] += y;
    }
  if (lane == 63)
#pragma unroll
    for (int i = 0; i < NV; ++i) lds[i][wave] = x[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int base = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) base += w < wave ? lds[i][w] : 0;
    tot[i] = lds[i][0] + lds[i][1] + lds[i][2] + lds[i][3];
    v[i] = base + x[i] - v[i];
  }
  __syncthreads();
}

// Rank of free slot t (stamp below `step`) by (stamp, slot) among the free
// slots; slots stamped `step` (the hits) sort after every free slot, so
// counting all slots below it suffices.  Writes q0[rank] = t; returns the
// rank, or -1 for a hit slot or t >= S.
__device__ __forceinline__ int rank_free_slot(const uint32_t *st, int S, uint32_t step, int32_t *q0) {
  const int t = threadIdx.x;
  if (t >= S || st[t] == step) return -1;
  const uint32_t k = st[t];
  int r = 0;
#pragma unroll 8
  for (int i = 0; i < S; ++i) {
    const uint32_t ki = st[i];
    r += (ki < k || (ki == k && i < t)) ? 1 : 0;
  }
  q0[r] = t;
  return r;
}

// Small batches.  Input: the batch's DecTile list (one tile per used expert,
// ascending expert; the host makes S at least its length, so it is batch 0
// alone).  Output: the fill list (expert, slot) of the misses and its range,
// counters, and every tile's expert field replaced by its slot.  Global
// stores come after the last barrier (a barrier would wait for them).
__global__ __launch_bounds__(256) void k_cache_plan(CacheState c, DecTile *__restrict__ dt,
                                                    const int32_t *__restrict__ ntile, int S, int E) {
  __shared__ uint32_t st[256];
  __shared__ int32_t q0[256], ml[256], es[256];
  __shared__ int scan_lds[2][4];
  const int t = threadIdx.x;
  const int n = *ntile;  // <= E <= 256
  const uint32_t step = c.hdr->step + 1u;
  const int e = t < n ? dt[t].e : -1;
  const int slot0 = e >= 0 ? c.expert_slot[e] : -1;
  const bool hit = slot0 >= 0, miss = e >= 0 && slot0 < 0;
  const int se_in = t < S ? c.slot_expert[t] : -1;
  st[t] = t < S ? c.stamp[t] : 0u;
  es[t] = -1;
  __syncthreads();
  if (hit) st[slot0] = step;  // distinct experts hold distinct slots
  int sv[2] = {miss ? 1 : 0, hit ? 1 : 0}, tot[2];
  block_scan<2>(sv, tot, scan_lds);
  const int m = sv[0], nm = tot[0], nhit = tot[1];
  const int room0 = S - nhit;
  const int r0 = nm > 0 ? rank_free_slot(st, S, step, q0) : -1;
  if (miss) ml[m] = e;
  __syncthreads();
  const int v = miss ? (m < room0 ? q0[m] : 0) : slot0;  // m < room0: S >= n, checked on the host
  int se_f = se_in;
  uint32_t st_f = t < S ? st[t] : 0u;
  if (r0 >= 0 && r0 < nm) {
    se_f = ml[r0];
    st_f = step;
  }
  if (t < S && se_f >= 0) es[se_f] = t;
  __syncthreads();
  if (miss) {
    c.fill_e[m] = e;
    c.fill_s[m] = v;
  }
  if (e >= 0) dt[t].e = v;
  if (t < S) {
    c.stamp[t] = st_f;
    c.slot_expert[t] = se_f;
  }
  if (t < E) c.expert_slot[t] = es[t];
  if (t == 0) {
    CacheHdr *h = c.hdr;
    c.frange[0] = 0;
    c.frange[1] = nm;
    h->step = step;
    h->fill_n = (uint32_t)nm;
    h->calls += 1ull;
    h->hits += (unsigned long long)nhit;
    h->misses += (unsigned long long)nm;
  }
}

// Prefill.  Input: the routing's per-expert counts and offsets.  Outputs:
// the fill list in batch order with each batch's range of it, each batch's
// tile count and first tile, and the tile list rewritten in batch order
// (experts ascending inside a batch, the tiles of an expert as the routing
// cut them) with each expert's slot in place of the expert.  An expert may
// lose its slot to a later batch of the same call: the kernels of its own
// batch have run by then (stream order).  Global stores come after the
// last barrier.
__global__ __launch_bounds__(256) void k_cache_plan_prefill(CacheState c, const int32_t *__restrict__ counts,
                                                            const int32_t *__restrict__ offsets,
                                                            TileT *__restrict__ tiles, int tile_n, int S, int E) {
  __shared__ uint32_t st[256];
  __shared__ int32_t q0[256], ml[256], es[256], bpre[257], ord[256], tst[256];
  __shared__ int32_t x_slot[256], x_off[256], x_cnt[256];  // per expert: slot, first position, count
  __shared__ int scan_lds[3][4];
  const int t = threadIdx.x;
  const uint32_t step0 = c.hdr->step + 1u;
  const int cnt = t < E ? counts[t] : 0;
  const int slot0 = t < E ? c.expert_slot[t] : -1;
  const bool hit = cnt > 0 && slot0 >= 0, miss = cnt > 0 && slot0 < 0;
  const int ntl = cnt > 0 ? (cnt + tile_n - 1) / tile_n : 0;
  const int se_in = t < S ? c.slot_expert[t] : -1;
  st[t] = t < S ? c.stamp[t] : 0u;
  es[t] = -1;
  x_off[t] = t < E ? offsets[t] : 0;
  x_cnt[t] = cnt;
  __syncthreads();
  if (hit) st[slot0] = step0;
  int sv[2] = {miss ? 1 : 0, hit ? 1 : 0}, tot[2];
  block_scan<2>(sv, tot, scan_lds);
  const int m = sv[0], nm = tot[0], nhit = tot[1];
  const int room0 = S - nhit;                  // misses batch 0 takes at most
  const int nB = nm > room0 ? nm - room0 : 0;  // misses of the later batches
  const int nb = (nhit + nm + S - 1) / S;      // batches (>= 1: every call uses an expert)
  const bool inA = hit || (miss && m < room0), inB = miss && m >= room0;
  const int r0 = nm > 0 ? rank_free_slot(st, S, step0, q0) : -1;
  if (miss) ml[m] = t;
  // tile order: batch 0's experts ascending, then the later batches' (their misses ascending)
  int pv[3] = {inA ? 1 : 0, inA ? ntl : 0, inB ? ntl : 0}, ptot[3];
  block_scan<3>(pv, ptot, scan_lds);  // its barriers also publish q0 and ml
  const int nA = ptot[0], tA = ptot[1], tB = ptot[2];
  const int v = miss ? (m < room0 ? q0[m] : (m - room0) % S) : slot0;
  x_slot[t] = cnt > 0 ? v : 0;
  if (cnt > 0) {
    const int r = inA ? pv[0] : nA + (m - room0);
    ord[r] = t;
    tst[r] = inA ? pv[1] : tA + pv[2];
  }
  if (inB) bpre[m - room0] = pv[2];
  if (t == 0) bpre[nB] = tB;
  // final slot contents: the last miss that took slot t, if any
  int se_f = se_in;
  uint32_t st_f = t < S ? st[t] : 0u;
  if (t < S) {
    int mf = -1;
    if (nb == 1) {
      if (r0 >= 0 && r0 < nm) {
        mf = r0;
        st_f = step0;
      }
    } else {
      const int szl = nB - (nb - 2) * S;  // misses of the last batch (1..S)
      if (t < szl) {
        mf = room0 + (nb - 2) * S + t;
        st_f = step0 + (uint32_t)(nb - 1);
      } else if (nb >= 3) {
        mf = room0 + (nb - 3) * S + t;
        st_f = step0 + (uint32_t)(nb - 2);
      } else {  // batch 0 took every free slot; hit slots keep their expert
        mf = r0;
        st_f = step0;
      }
    }
    if (mf >= 0) se_f = ml[mf];
    if (se_f >= 0) es[se_f] = t;
  }
  __syncthreads();
  if (miss) {
    c.fill_e[m] = t;
    c.fill_s[m] = v;
  }
  if (t < E) {  // batch t
    int cj = 0, first = 0, f0 = nm, f1 = nm;
    if (t == 0) {
      cj = tA;
      f0 = 0;
      f1 = nm < room0 ? nm : room0;
    } else if (t < nb) {
      const int b0 = (t - 1) * S, b1 = t * S < nB ? t * S : nB;
      first = tA + bpre[b0];
      cj = bpre[b1] - bpre[b0];
      f0 = room0 + b0;
      f1 = room0 + b1;
    }
    c.brange[2 * t] = cj;
    c.brange[2 * t + 1] = first;
    c.frange[2 * t] = f0;
    c.frange[2 * t + 1] = f1;
    c.expert_slot[t] = es[t];
  }
  if (t < S) {
    c.stamp[t] = st_f;
    c.slot_expert[t] = se_f;
  }
  if (t == 0) {
    CacheHdr *h = c.hdr;
    h->step = step0 + (uint32_t)(nb - 1);
    h->fill_n = (uint32_t)nm;
    h->calls += 1ull;
    h->hits += (unsigned long long)nhit;
    h->misses += (unsigned long long)nm;
  }
  // the tiles: tile i belongs to the last expert (in tile order) starting at or before it
  const int U = nhit + nm, ntot = tA + tB;
  for (int i = t; i < ntot; i += 256) {
    int lo = 0, hi = U - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tst[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const int x = ord[lo], li = i - tst[lo];
    TileT tl;
    tl.e = x_slot[x];
    tl.p0 = x_off[x] + li * tile_n;
    tl.n = min(tile_n, x_cnt[x] - li * tile_n);
    tl.pad = 0;
    tiles[i] = tl;
  }
}

// Copy fill items [fr[0], fr[1]) from host memory into their slots: workgroup
// (item, chunk) moves CACHE_CHUNK bytes of the item's gate | up | down bytes
// (16-byte words; every matrix is a multiple of 16 bytes).  Workgroups past
// the range return at once.
constexpr int CACHE_CHUNK = 65536;

__global__ __launch_bounds__(256) void k_cache_fill(CacheState c, const int32_t *__restrict__ fr,
                                                    const uint8_t *__restrict__ hg, const uint8_t *__restrict__ hu,
                                                    const uint8_t *__restrict__ hd, uint64_t gu_bytes,
                                                    uint64_t d_bytes, int chunks) {
  const int item = fr[0] + (int)(blockIdx.x / chunks);
  const int chunk = blockIdx.x % chunks;
  if (item >= fr[1]) return;  // uniform
  const int e = c.fill_e[item], s = c.fill_s[item];
  const uint64_t total = 2 * gu_bytes + d_bytes;
  const uint64_t b0 = (uint64_t)chunk * CACHE_CHUNK;
  constexpr int PER = CACHE_CHUNK / (256 * 16);  // 16-byte words per thread
  u4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {  // all loads first: host reads have long latency
    const uint64_t b = b0 + 16ull * (threadIdx.x + 256 * i);
    if (b < total) {
      const uint8_t *src = b < gu_bytes ? hg + (uint64_t)e * gu_bytes + b
                           : b < 2 * gu_bytes ? hu + (uint64_t)e * gu_bytes + (b - gu_bytes)
                                              : hd + (uint64_t)e * d_bytes + (b - 2 * gu_bytes);
      v[i] = *reinterpret_cast<const u4 *>(src);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint64_t b = b0 + 16ull * (threadIdx.x + 256 * i);
    if (b < total) {
      uint8_t *dst = b < gu_bytes ? c.gate + (uint64_t)s * gu_bytes + b
                     : b < 2 * gu_bytes ? c.up + (uint64_t)s * gu_bytes + (b - gu_bytes)
                                        : c.down + (uint64_t)s * d_bytes + (b - 2 * gu_bytes);
      *reinterpret_cast<u4 *>(dst) = v[i];
    }
  }
}

hipError_t launch_cache_reset(const CacheState &c, int S, int E, hipStream_t s) {
  hipLaunchKernelGGL(k_cache_reset, dim3(1), dim3(256), 0, s, c, S, E);
  return hipGetLastError();
}

hipError_t launch_cache_plan(const CacheState &c, DecTile *dt, const int32_t *ntile, int S, int E, hipStream_t s,
                             const Timing *tm) {
  DS4_LAUNCH(tm, k_cache_plan, dim3(1), dim3(256), 0, s, c, dt, ntile, S, E);
  return hipGetLastError();
}

hipError_t launch_cache_plan_prefill(const CacheState &c, const int32_t *counts, const int32_t *offsets,
                                     TileT *tiles, int tile_n, int S, int E, hipStream_t s) {
  hipLaunchKernelGGL(k_cache_plan_prefill, dim3(1), dim3(256), 0, s, c, counts, offsets, tiles, tile_n, S, E);
  return hipGetLastError();
}

hipError_t launch_cache_fill(const CacheState &c, const int32_t *fr, const void *hg, const void *hu, const void *hd,
                             size_t gu_bytes, size_t d_bytes, int max_items, hipStream_t s, const Timing *tm) {
  if (max_items <= 0) return hipSuccess;
  const uint64_t total = 2 * (uint64_t)gu_bytes + d_bytes;
  const int chunks = (int)((total + CACHE_CHUNK - 1) / CACHE_CHUNK);
  DS4_LAUNCH(tm, k_cache_fill, dim3((unsigned)((int64_t)max_items * chunks)), dim3(256), 0, s, c, fr,
             (const uint8_t *)hg, (const uint8_t *)hu, (const uint8_t *)hd, (uint64_t)gu_bytes, (uint64_t)d_bytes,
             chunks);
  return hipGetLastError();
}

}  // namespace ds4
