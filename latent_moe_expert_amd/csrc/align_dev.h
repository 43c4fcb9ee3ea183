// Device pieces of moe_align_block_size shared by the align kernels and the fused decode
// route + align kernel (layout defined in align.hip).
#pragma once
#include "common.h"

namespace moe {

constexpr int kChunk = 64;  // tokens per chunk (one bit each in a 64-bit mask)

// Slots of a chunk whose ids are also staged in LDS (for the repeat check below).
constexpr int kIdsLds = 4096;

// The chunk's 64-bit token masks per expert; with ids_l, also the chunk's ids (when the chunk
// has at most kIdsLds slots).
__device__ __forceinline__ void build_masks(const int32_t* __restrict__ ids, int T, int k, int E, int chunk,
                                            unsigned long long* mask, int32_t* ids_l) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
  __syncthreads();
  const int t0 = chunk * kChunk;
  const int nt = min(kChunk, T - t0);
  const int np = nt * k;
  const bool stage = ids_l != nullptr && np <= kIdsLds;
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    const int e = ids[(size_t)t0 * k + i];
    if (stage) ids_l[i] = e;
    if (e >= 0 && e < E) atomicOr(&mask[e], 1ull << (i / k));
  }
  __syncthreads();
}

// true when slot j of a token repeats the id of an earlier slot of the same token; tok_l
// (LDS) or tok (global) point at the token's first slot. The LDS copy keeps the up to k - 1
// dependent reads off the memory path.
__device__ __forceinline__ bool repeated_in_token(const int32_t* tok_l, const int32_t* __restrict__ tok, bool staged,
                                                  int j, int e) {
  if (staged) {
    for (int u = 0; u < j; ++u)
      if (tok_l[u] == e) return true;
  } else {
    for (int u = 0; u < j; ++u)
      if (tok[u] == e) return true;
  }
  return false;
}

// Many experts (their per-expert LDS masks would not fit): the chunk's masks live in an LDS hash
// table keyed by expert id. A chunk of 64 tokens with k <= 64 lists at most 4096 distinct experts,
// so the table (8192 slots, linear probing) is at most half full and every probe sequence ends.
constexpr int kHashSlots = 8192;
constexpr int kLdsExperts = 4096;  // up to this many experts the masks are an LDS array indexed by expert

// slot of expert e, inserting it if absent (-1 never happens for k <= 64)
__device__ __forceinline__ int hash_slot(int32_t* keys, int e) {
  uint32_t h = ((uint32_t)e * 2654435761u) >> 19;  // 13 bits
  for (int p = 0; p < kHashSlots; ++p) {
    const int old = atomicCAS(&keys[h], -1, e);
    if (old == -1 || old == e) return (int)h;
    h = (h + 1) & (kHashSlots - 1);
  }
  return -1;
}

__device__ __forceinline__ void build_masks_hash(const int32_t* __restrict__ ids, int T, int k, int E, int chunk,
                                                 int32_t* keys, unsigned long long* masks, int32_t* ids_l) {
  for (int i = threadIdx.x; i < kHashSlots; i += blockDim.x) {
    keys[i] = -1;
    masks[i] = 0ull;
  }
  __syncthreads();
  const int t0 = chunk * kChunk;
  const int nt = min(kChunk, T - t0);
  const int np = nt * k;
  const bool stage = ids_l != nullptr && np <= kIdsLds;
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    const int e = ids[(size_t)t0 * k + i];
    if (stage) ids_l[i] = e;
    if (e >= 0 && e < E) {
      const int h = hash_slot(keys, e);
      if (h >= 0) atomicOr(&masks[h], 1ull << (i / k));
    }
  }
  __syncthreads();
}

// Exclusive prefix sum of v over the NT threads of the block (thread order), and the block's
// total: an inclusive scan inside each wave, the wave totals through part (NT / 64 entries),
// one block barrier. Integer sums: the order of additions does not change the result.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* part, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d, 64);
    if (lane >= d) incl += u;
  }
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int u = part[w];
    before += w < wave ? u : 0;
    all += u;
  }
  *total = all;
  return before + incl - v;
}

// All T <= 64 * nc tokens in one block of NT threads: the nc chunks' masks, counts, the scan
// over experts, padding and scatter. mask holds nc * E entries (chunk-major), offs E, part NT,
// ids_l kIdsLds. A slot's rank inside its expert is the popcounts of the earlier chunks' masks
// plus popcount(mask & lower tokens) in its own chunk, as in the multi-block form.
template <int NT>
__device__ __forceinline__ void align_chunks(const int32_t* __restrict__ ids, int T, int k, int E, int B, int cap,
                                             int nc, int32_t* __restrict__ counts, int32_t* __restrict__ sorted_ids,
                                             int32_t* __restrict__ expert_ids, int32_t* __restrict__ num_post,
                                             int32_t* __restrict__ inv_pos, unsigned long long* mask, int* offs,
                                             int* part, int32_t* ids_l) {
  const int tid = threadIdx.x;
  const int pairs = T * k;
  const bool stage = pairs <= kIdsLds;
  for (int i = tid; i < nc * E; i += NT) mask[i] = 0ull;
  __syncthreads();
  for (int i = tid; i < pairs; i += NT) {
    const int e = ids[i];
    if (stage) ids_l[i] = e;
    const int t = i / k;
    if (e >= 0 && e < E) atomicOr(&mask[(t >> 6) * E + e], 1ull << (t & 63));
  }
  __syncthreads();
  const int per = (E + NT - 1) / NT;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) {
    int c = 0;
    for (int q = 0; q < nc; ++q) c += __popcll(mask[q * E + e]);
    counts[e] = c;
    local += (c + B - 1) / B * B;
  }
  int total;
  int run = block_exclusive_scan<NT>(local, part, &total);
  for (int e = e0; e < e1; ++e) {
    offs[e] = run;
    int c = 0;
    for (int q = 0; q < nc; ++q) c += __popcll(mask[q * E + e]);
    const int p = (c + B - 1) / B * B;
    for (int b = 0; b < p / B; ++b) expert_ids[run / B + b] = e;
    for (int i = c; i < p; ++i) sorted_ids[run + i] = pairs;
    run += p;
  }
  if (tid == 0) *num_post = total;
  for (int i = total + tid; i < cap; i += NT) sorted_ids[i] = pairs;
  for (int b = total / B + tid; b < cap / B; b += NT) expert_ids[b] = -1;
  __syncthreads();
  for (int i = tid; i < pairs; i += NT) {
    const int e = stage ? ids_l[i] : ids[i];
    const int t = i / k;
    if (e < 0 || e >= E || repeated_in_token(ids_l + t * k, ids + (size_t)t * k, stage, i - t * k, e)) {
      inv_pos[i] = -1;
      continue;
    }
    const int q = t >> 6, tl = t & 63;
    int pos = offs[e];
    for (int u = 0; u < q; ++u) pos += __popcll(mask[u * E + e]);
    pos += tl ? __popcll(mask[q * E + e] & ((1ull << tl) - 1ull)) : 0;
    sorted_ids[pos] = i;
    inv_pos[i] = pos;
  }
}

}  // namespace moe
