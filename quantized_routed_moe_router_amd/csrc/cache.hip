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

// One workgroup.  Input: the batch's DecTile list (one tile per used expert,
// ascending expert).  Hits take the current step as their stamp first, so no
// expert of the batch is evicted; then each miss, in tile order, takes the
// slot with the oldest stamp (ties: the lower slot), evicting its expert.
// Output: the fill list (expert, slot) of the misses, counters, and every
// tile's expert field replaced by its slot.
__global__ __launch_bounds__(256) void k_cache_plan(CacheState c, DecTile *__restrict__ dt,
                                                    const int32_t *__restrict__ ntile, int S, int E) {
  __shared__ uint32_t st[256];
  __shared__ int32_t se[256], es[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = *ntile;
  const uint32_t step = c.hdr->step + 1u;
  for (int s = tid; s < 256; s += 256) {
    st[s] = s < S ? c.stamp[s] : 0u;
    se[s] = s < S ? c.slot_expert[s] : -1;
  }
  for (int e = tid; e < 256; e += 256) es[e] = e < E ? c.expert_slot[e] : -1;
  __syncthreads();
  if (tid < n) {  // distinct experts per tile: no two threads stamp one slot
    const int s = es[dt[tid].e];
    if (s >= 0) st[s] = step;
  }
  __syncthreads();
  if (tid < 64) {
    int nf = 0;
    for (int i = 0; i < n; ++i) {
      const int e = dt[i].e;  // uniform
      if (es[e] >= 0) continue;
      // victim: smallest (stamp, slot) among slots not used by this batch
      uint64_t key = ~0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = lane + 64 * j;
        if (s < S && st[s] != step) {
          const uint64_t k = ((uint64_t)st[s] << 32) | (uint32_t)s;
          key = k < key ? k : key;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t k = __shfl_xor(key, o);
        key = k < key ? k : key;
      }
      // a victim exists (S >= distinct experts of the batch, checked on the host)
      if (key == ~0ull) break;
      const int v = (int)(uint32_t)key;
      if (lane == 0) {
        const int old = se[v];
        if (old >= 0) es[old] = -1;
        se[v] = e;
        es[e] = v;
        st[v] = step;
        c.fill_e[nf] = e;
        c.fill_s[nf] = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      ++nf;
    }
    if (lane == 0) {
      CacheHdr *h = c.hdr;
      c.frange[0] = 0;
      c.frange[1] = nf;
      h->step = step;
      h->fill_n = (uint32_t)nf;
      h->calls += 1ull;
      h->hits += (unsigned long long)(n - nf);
      h->misses += (unsigned long long)nf;
    }
  }
  __syncthreads();
  if (tid < n) dt[tid].e = es[dt[tid].e];
  for (int s = tid; s < S; s += 256) {
    c.stamp[s] = st[s];
    c.slot_expert[s] = se[s];
  }
  for (int e = tid; e < E; e += 256) c.expert_slot[e] = es[e];
}

// Prefill through the cache.  One workgroup (E <= 256).  The experts the
// call uses (count > 0) go through the slots in batches of at most S: batch 0
// holds every hit and then misses in ascending expert order while slots
// remain, each later batch the next S misses.  Batch j has the stamp
// step+1+j, and inside it each miss, in ascending order, takes the slot with
// the oldest stamp (ties: the lower slot) among the slots the batch has not
// taken: the small-batch plan above, batch after batch.  A victim always
// exists: a batch holds at most S experts and every older stamp is below its
// own.  Outputs: the fill list in batch order with each batch's range of it,
// each batch's tile count and first tile, and the tile list rewritten in
// batch order (experts ascending inside a batch) with each expert's slot in
// place of the expert.  A batch's expert may lose its slot to a later batch:
// the kernels of its batch have run by then (stream order).
__global__ __launch_bounds__(256) void k_cache_plan_prefill(CacheState c, const int32_t *__restrict__ counts,
                                                            const int32_t *__restrict__ offsets,
                                                            TileT *__restrict__ tiles, int tile_n, int S, int E) {
  __shared__ uint32_t st[256];
  __shared__ int32_t se[256], es[256], cn[256], off[256], nt[256], eb[256], bs[256], ts[256], ml[256], bcnt[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t step0 = c.hdr->step + 1u;
  st[tid] = tid < S ? c.stamp[tid] : 0u;
  se[tid] = tid < S ? c.slot_expert[tid] : -1;
  const int cnt = tid < E ? counts[tid] : 0;
  const int slot0 = tid < E ? c.expert_slot[tid] : -1;
  const bool hit = cnt > 0 && slot0 >= 0;
  es[tid] = slot0;
  cn[tid] = cnt;
  off[tid] = tid < E ? offsets[tid] : 0;
  nt[tid] = cnt > 0 ? (cnt + tile_n - 1) / tile_n : 0;
  eb[tid] = hit ? 0 : -1;
  bs[tid] = hit ? slot0 : -1;
  bcnt[tid] = 0;
  __syncthreads();
  if (hit) st[slot0] = step0;  // distinct experts hold distinct slots
  const int nhit = __syncthreads_count(hit);
  const int nused = __syncthreads_count(cnt > 0);
  const int nm = nused - nhit;
  const int room0 = S - nhit;  // misses that fit batch 0
  const int nb = (nused + S - 1) / S;
  if (tid < 64) {
    // the misses in ascending order
    int base = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 64 * q + lane;
      const bool miss = nt[e] > 0 && eb[e] < 0;
      const uint64_t m = __ballot(miss);
      if (miss) ml[base + __popcll(m & ((1ull << lane) - 1ull))] = e;
      base += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    for (int m = 0; m < nm; ++m) {
      const int e = ml[m];  // uniform
      const int j = m < room0 ? 0 : 1 + (m - room0) / S;
      const uint32_t step = step0 + (uint32_t)j;
      uint64_t key = ~0ull;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = lane + 64 * i;
        if (s < S && st[s] != step) {
          const uint64_t k = ((uint64_t)st[s] << 32) | (uint32_t)s;
          key = k < key ? k : key;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t k = __shfl_xor(key, o);
        key = k < key ? k : key;
      }
      if (key == ~0ull) break;  // not reached (see above); keeps LDS indexes in range
      const int v = (int)(uint32_t)key;
      if (lane == 0) {
        const int old = se[v];
        if (old >= 0) es[old] = -1;
        se[v] = e;
        es[e] = v;
        st[v] = step;
        eb[e] = j;
        bs[e] = v;
        c.fill_e[m] = e;
        c.fill_s[m] = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
  __syncthreads();
  // first tile of each expert: tiles of the experts before it in (batch, expert) order
  const int e = tid;
  if (nt[e] > 0) {
    const int key = eb[e] * 256 + e;
    int t0 = 0;
    for (int i = 0; i < 256; ++i) t0 += (nt[i] > 0 && eb[i] * 256 + i < key) ? nt[i] : 0;
    ts[e] = t0;
    if (eb[e] >= 0) atomicAdd(&bcnt[eb[e]], nt[e]);
  }
  __syncthreads();
  if (tid < E) {
    const int j = tid;
    int first = 0;
    for (int i = 0; i < j; ++i) first += bcnt[i];
    c.brange[2 * j] = bcnt[j];
    c.brange[2 * j + 1] = first;
    const int f0 = j == 0 ? 0 : min(nm, room0 + (j - 1) * S), f1 = min(nm, room0 + j * S);
    c.frange[2 * j] = j < nb ? f0 : nm;
    c.frange[2 * j + 1] = j < nb ? f1 : nm;
  }
  for (int x = 0; x < E; ++x) {  // uniform
    const int n = nt[x];
    const int slot = bs[x] >= 0 ? bs[x] : 0;
    for (int i = tid; i < n; i += 256) {
      TileT tl;
      tl.e = slot;
      tl.p0 = off[x] + i * tile_n;
      tl.n = min(tile_n, cn[x] - i * tile_n);
      tl.pad = 0;
      tiles[ts[x] + i] = tl;
    }
  }
  if (tid < S) {
    c.stamp[tid] = st[tid];
    c.slot_expert[tid] = se[tid];
  }
  if (tid < E) c.expert_slot[tid] = es[tid];
  if (tid == 0) {
    CacheHdr *h = c.hdr;
    h->step = step0 + (uint32_t)(nb > 0 ? nb - 1 : 0);
    h->fill_n = (uint32_t)nm;
    h->calls += 1ull;
    h->hits += (unsigned long long)nhit;
    h->misses += (unsigned long long)nm;
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
