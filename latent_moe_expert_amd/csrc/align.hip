// moe_align_block_size: the padded, expert-sorted layout of (token, slot) pairs
// that the grouped expert contractions read (SlimServe quants.md, note on the
// alignment fix: one layout whose rows are aligned to the LCM of the consumers'
// tile widths, with an expert id per tile; expert ids above 255 must work).
//
// Layout produced (bit-exact, integer only):
//   sorted_ids: for experts in ascending id order, the flat slot indices t*k+j
//               that chose the expert, ascending, then padding with the
//               sentinel T*k up to a multiple of B; empty experts get nothing;
//               the tail up to capacity holds the sentinel.
//   expert_ids: expert of each block of B entries, -1 past the end.
//   num_post:   padded entry count; inv_pos[t*k+j] = position of that slot.
//
// Three kernels, no float and no order-dependent atomics:
//   count   one block per chunk of 64 tokens builds, in LDS, a 64-bit mask per
//           expert of the chunk tokens that chose it; writes popcounts.
//   scan    one block: per-expert prefix over chunks, padded sizes, the
//           exclusive scan over experts, expert_ids and all padding.
//   scatter one block per chunk rebuilds the masks; a slot's rank inside its
//           expert is (chunk prefix) + popcount(mask & lower tokens).
// Above 4096 experts the per-expert masks of a chunk do not fit LDS as an array indexed by
// expert; they are kept in an LDS hash table of the experts the chunk's tokens list (at most
// 64 * k <= 4096 of them in 8192 slots), with the same counts, scan and ranks.
// Each token lists an expert at most once (the router's ids are distinct), so
// token order inside an expert equals flat-index order. An id a token repeats is
// kept at its first slot only; the later slots are treated like ids out of range
// (no entry, inv_pos -1), so the result is still deterministic.
#include "align_dev.h"
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void align_count_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                          int32_t* __restrict__ chunk_cnt) {
  extern __shared__ unsigned long long mask[];
  build_masks(ids, T, k, E, blockIdx.x, mask, nullptr);
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    chunk_cnt[(size_t)blockIdx.x * E + e] = __popcll(mask[e]);
}

__global__ __launch_bounds__(1024) void align_scan_kernel(int nchunks, int E, int B, int pairs, int cap,
                                                          int32_t* __restrict__ chunk_cnt /* in: counts, out: prefix */,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offs,
                                                          int32_t* __restrict__ sorted_ids,
                                                          int32_t* __restrict__ expert_ids,
                                                          int32_t* __restrict__ num_post) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  // per-expert prefix over chunks, 16 chunks' loads in flight at a time (a load past the
  // last chunk reads zero from the buffer resource, so none of them sits under a branch)
  constexpr int kBatch = 16;
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      // this batch's rows only (kBatch * E * 4 bytes < 2^32 for E <= 65535)
      const __amdgpu_buffer_rsrc_t cc =
          make_rsrc(chunk_cnt + (size_t)c0 * E, (uint32_t)min(kBatch, nchunks - c0) * (uint32_t)E * 4u);
      int v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b32(cc, ((uint32_t)u * (uint32_t)E + (uint32_t)e) * 4u, 0, 0);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (c0 + u < nchunks) chunk_cnt[(size_t)(c0 + u) * E + e] = run;
        run += v[u];
      }
    }
    counts[e] = run;
  }
  __syncthreads();
  // exclusive scan of padded sizes over experts: thread tid owns a contiguous run
  const int per = (E + 1023) / 1024;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += (counts[e] + B - 1) / B * B;
  int total;
  int run = block_exclusive_scan<1024>(local, part, &total);
  for (int e = e0; e < e1; ++e) {
    offs[e] = run;
    run += (counts[e] + B - 1) / B * B;
  }
  if (tid == 0) *num_post = total;
  __syncthreads();
  // expert ids per block and padding entries of each segment
  for (int e = tid; e < E; e += 1024) {
    const int c = counts[e];
    const int p = (c + B - 1) / B * B;
    const int o = offs[e];
    for (int b = 0; b < p / B; ++b) expert_ids[o / B + b] = e;
    for (int i = c; i < p; ++i) sorted_ids[o + i] = pairs;
  }
  for (int i = total + tid; i < cap; i += 1024) sorted_ids[i] = pairs;
  for (int b = total / B + tid; b < cap / B; b += 1024) expert_ids[b] = -1;
}

__global__ __launch_bounds__(256) void align_scatter_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                            const int32_t* __restrict__ chunk_pre,
                                                            const int32_t* __restrict__ offs,
                                                            int32_t* __restrict__ sorted_ids,
                                                            int32_t* __restrict__ inv_pos) {
  extern __shared__ unsigned long long mask[];
  __shared__ int32_t ids_l[kIdsLds];
  build_masks(ids, T, k, E, blockIdx.x, mask, ids_l);
  const int t0 = blockIdx.x * kChunk;
  const int nt = min(kChunk, T - t0);
  const int np = nt * k;
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    const int flat = t0 * k + i;
    const int e = ids[flat];
    const int tl = i / k;
    if (e < 0 || e >= E ||
        repeated_in_token(ids_l + tl * k, ids + (size_t)(t0 + tl) * k, np <= kIdsLds, i - tl * k, e)) {
      inv_pos[flat] = -1;
      continue;
    }
    const unsigned long long below = tl ? (mask[e] & ((1ull << tl) - 1ull)) : 0ull;
    const int pos = offs[e] + chunk_pre[(size_t)blockIdx.x * E + e] + __popcll(below);
    sorted_ids[pos] = flat;
    inv_pos[flat] = pos;
  }
}

// Count and scatter for many experts (E > kLdsExperts): the same per-chunk masks, kept in the
// LDS hash table; the count kernel first clears its chunk's row of counts (experts absent from
// the chunk keep 0).
__global__ __launch_bounds__(256) void align_count_hash_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                               int32_t* __restrict__ chunk_cnt) {
  __shared__ int32_t keys[kHashSlots];
  __shared__ unsigned long long masks[kHashSlots];
  int32_t* row = chunk_cnt + (size_t)blockIdx.x * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) row[e] = 0;
  build_masks_hash(ids, T, k, E, blockIdx.x, keys, masks, nullptr);  // its barriers order the clears first
  for (int h = threadIdx.x; h < kHashSlots; h += blockDim.x)
    if (keys[h] >= 0) row[keys[h]] = __popcll(masks[h]);
}

__global__ __launch_bounds__(256) void align_scatter_hash_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                                 const int32_t* __restrict__ chunk_pre,
                                                                 const int32_t* __restrict__ offs,
                                                                 int32_t* __restrict__ sorted_ids,
                                                                 int32_t* __restrict__ inv_pos) {
  __shared__ int32_t keys[kHashSlots];
  __shared__ unsigned long long masks[kHashSlots];
  __shared__ int32_t ids_l[kIdsLds];
  build_masks_hash(ids, T, k, E, blockIdx.x, keys, masks, ids_l);
  const int t0 = blockIdx.x * kChunk;
  const int nt = min(kChunk, T - t0);
  const int np = nt * k;
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    const int flat = t0 * k + i;
    const int e = ids[flat];
    const int tl = i / k;
    if (e < 0 || e >= E ||
        repeated_in_token(ids_l + tl * k, ids + (size_t)(t0 + tl) * k, np <= kIdsLds, i - tl * k, e)) {
      inv_pos[flat] = -1;
      continue;
    }
    const int h = hash_slot(keys, e);  // present: found, not inserted
    if (h < 0) {                       // not reached for k <= 64 (the table stays half empty)
      inv_pos[flat] = -1;
      continue;
    }
    const unsigned long long below = tl ? (masks[h] & ((1ull << tl) - 1ull)) : 0ull;
    const int pos = offs[e] + chunk_pre[(size_t)blockIdx.x * E + e] + __popcll(below);
    sorted_ids[pos] = flat;
    inv_pos[flat] = pos;
  }
}

// Batches of up to kFewChunks chunks (T <= 64 * kFewChunks) in a single block: masks, counts,
// scan, padding and scatter, so small batches pay one launch instead of three.
constexpr int kFewChunks = 8;
constexpr size_t kFewLds = 64 * 1024;  // dynamic LDS for the masks and the expert offsets

__global__ __launch_bounds__(1024) void align_single_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                            int B, int cap, int nc, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ sorted_ids,
                                                            int32_t* __restrict__ expert_ids,
                                                            int32_t* __restrict__ num_post,
                                                            int32_t* __restrict__ inv_pos) {
  extern __shared__ unsigned long long mask[];      // [nc * E]
  int* offs = (int*)(mask + (size_t)nc * E);         // [E]
  __shared__ int part[1024];
  __shared__ int32_t ids_l[kIdsLds];
  align_chunks<1024>(ids, T, k, E, B, cap, nc, counts, sorted_ids, expert_ids, num_post, inv_pos, mask, offs, part,
                     ids_l);
}

}  // namespace

int align_capacity(int T, int k, int E, int B) {
  const long long pairs = (long long)T * k;
  const long long d = pairs < E ? pairs : E;
  return (int)(B * ((pairs + d * (B - 1)) / B));
}

size_t align_scratch_bytes(int T, int E) {
  const size_t nchunks = (size_t)(T + kChunk - 1) / kChunk;
  return (nchunks * E + E) * sizeof(int32_t);  // chunk prefixes + expert offsets
}

hipError_t launch_align(const int32_t* ids, int T, int k, int E, int B, int32_t* counts, int32_t* sorted_ids,
                        int32_t* expert_ids, int32_t* num_post, int32_t* inv_pos, void* scratch, hipStream_t s) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int cap = align_capacity(T, k, E, B);
  int32_t* chunk = (int32_t*)scratch;
  int32_t* offs = chunk + (size_t)nchunks * E;
  const size_t lds = (size_t)E * sizeof(unsigned long long);
  if (E > kLdsExperts) {  // masks in an LDS hash table (k <= 64)
    if (k > 64) return hipErrorInvalidValue;
    if (nchunks > 0) hipLaunchKernelGGL(align_count_hash_kernel, dim3(nchunks), dim3(256), 0, s, ids, T, k, E, chunk);
    hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(1024), 0, s, nchunks, E, B, T * k, cap, chunk, counts, offs,
                       sorted_ids, expert_ids, num_post);
    if (nchunks > 0)
      hipLaunchKernelGGL(align_scatter_hash_kernel, dim3(nchunks), dim3(256), 0, s, ids, T, k, E, chunk, offs,
                         sorted_ids, inv_pos);
    return hipGetLastError();
  }
  const size_t few = (size_t)nchunks * lds + (size_t)E * sizeof(int);
  if (nchunks <= 1 || (nchunks <= kFewChunks && few <= kFewLds)) {
    const int nc = nchunks > 1 ? nchunks : 1;
    hipLaunchKernelGGL(align_single_kernel, dim3(1), dim3(1024), (size_t)nc * lds + (size_t)E * sizeof(int), s, ids,
                       T, k, E, B, cap, nc, counts, sorted_ids, expert_ids, num_post, inv_pos);
    return hipGetLastError();
  }
  if (nchunks > 0) hipLaunchKernelGGL(align_count_kernel, dim3(nchunks), dim3(256), lds, s, ids, T, k, E, chunk);
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(1024), 0, s, nchunks, E, B, T * k, cap, chunk, counts, offs,
                     sorted_ids, expert_ids, num_post);
  if (nchunks > 0)
    hipLaunchKernelGGL(align_scatter_kernel, dim3(nchunks), dim3(256), lds, s, ids, T, k, E, chunk, offs,
                       sorted_ids, inv_pos);
  return hipGetLastError();
}

}  // namespace moe
