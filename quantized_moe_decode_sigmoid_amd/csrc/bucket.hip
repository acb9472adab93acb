// Token-to-expert bucketing: histogram, exclusive prefix sum and a stable
// permutation of the routes grouped by expert (PocketLLM design record,
// section 4: the routes are sorted by expert so that every output element has
// exactly one writer and the top-k can be summed in slot order afterwards).
//
// One workgroup of 1024 threads (16 wavefronts).  Integer work only, so the
// result is bit-exact whatever the scheduling:
//   1. counts by LDS atomic increments (the totals do not depend on order);
//   2. exclusive scan over the (at most 256) experts;
//   3. routes taken 1024 at a time in route order; inside a wavefront, the
//      lanes holding the same expert find each other with 8 ballots (one per
//      bit of the expert id) and rank themselves by lane; per-wave counts in
//      LDS give the offset of each wavefront; a running offset per expert
//      carries across tiles.  Position = running + earlier waves + lane rank,
//      which is exactly the stable order (ascending route id in an expert).
// The same pass writes the work list of the FFN kernels: chunks of at most
// chunk_rows routes of one expert, then chunks of chunk_rows tokens of the
// shared expert (chunk_rows is a power of two).
#include "device.h"
#include "launch.h"

namespace qmoe {

constexpr int kBucketThreads = 1024;
constexpr int kBucketWaves = kBucketThreads / 64;

__global__ __launch_bounds__(kBucketThreads) void k_bucket(const int32_t* __restrict__ ids, int T, int K, int E,
                                                           int n_shared, int chunk_shift, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ pos, Chunk* __restrict__ chunks,
                                                           int32_t* __restrict__ n_chunks) {
  __shared__ int32_t s_cnt[256];
  __shared__ int32_t s_run[256];
  __shared__ int32_t s_wave[kBucketWaves][256];
  __shared__ int32_t s_chunk_first[257];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int R = T * K;

  for (int e = tid; e < 256; e += kBucketThreads) s_cnt[e] = 0;
  __syncthreads();
  for (int r = tid; r < R; r += kBucketThreads) atomicAdd(&s_cnt[ids[r]], 1);
  __syncthreads();
  if (tid == 0) {
    int run = 0, ch = 0;
    for (int e = 0; e < E; e++) {
      s_run[e] = run;
      s_chunk_first[e] = ch;
      run += s_cnt[e];
      ch += (s_cnt[e] + (1 << chunk_shift) - 1) >> chunk_shift;
    }
    s_chunk_first[E] = ch;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kBucketThreads) {
    counts[e] = s_cnt[e];
    offsets[e] = s_run[e];
  }
  if (tid == 0) offsets[E] = R;

  // chunk list (independent of the permutation itself); optional
  const bool want_chunks = chunks != nullptr;
  for (int e = tid; want_chunks && e < E; e += kBucketThreads) {
    const int rows = 1 << chunk_shift;
    const int c0 = s_chunk_first[e], nch = (s_cnt[e] + rows - 1) >> chunk_shift;
    for (int j = 0; j < nch; j++) {
      Chunk c;
      c.expert = e;
      c.first = s_run[e] + rows * j;
      c.count = min(rows, s_cnt[e] - rows * j);
      c.pad = 0;
      chunks[c0 + j] = c;
    }
  }
  const int routed_chunks = s_chunk_first[E];
  const int shared_chunks = n_shared ? (T + (1 << chunk_shift) - 1) >> chunk_shift : 0;
  for (int j = tid; want_chunks && j < shared_chunks; j += kBucketThreads) {
    Chunk c;
    c.expert = -1;
    c.first = j << chunk_shift;
    c.count = min(1 << chunk_shift, T - (j << chunk_shift));
    c.pad = 0;
    chunks[routed_chunks + j] = c;
  }
  if (tid == 0 && want_chunks) *n_chunks = routed_chunks + shared_chunks;

  // stable scatter
  for (int base = 0; base < R; base += kBucketThreads) {
    const int r = base + tid;
    const bool valid = r < R;
    const int key = valid ? ids[r] : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; bit++) {
      const uint64_t b = __ballot(valid && ((key >> bit) & 1));
      peers &= ((key >> bit) & 1) ? b : ~b;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & below);
    for (int i = tid; i < kBucketWaves * 256; i += kBucketThreads) (&s_wave[0][0])[i] = 0;
    __syncthreads();
    if (valid && rank == 0) s_wave[wave][key] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int before = 0;
      for (int w = 0; w < wave; w++) before += s_wave[w][key];
      const int at = s_run[key] + before + rank;
      perm[at] = r;
      if (pos) pos[r] = at;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kBucketThreads) {
      int tot = 0;
      for (int w = 0; w < kBucketWaves; w++) tot += s_wave[w][e];
      s_run[e] += tot;
    }
    __syncthreads();
  }
}

hipError_t launch_bucket(const int32_t* ids, int T, int K, int E, int n_shared, int chunk_rows, int32_t* counts,
                         int32_t* offsets, int32_t* perm, int32_t* pos, Chunk* chunks, int32_t* n_chunks,
                         hipStream_t stream) {
  int shift = 0;
  while ((1 << shift) < chunk_rows) shift++;
  clear_last_error();
  hipLaunchKernelGGL(k_bucket, dim3(1), dim3(kBucketThreads), 0, stream, ids, T, K, E, n_shared, shift, counts,
                     offsets, perm, pos, chunks, n_chunks);
  return hipGetLastError();
}

}  // namespace qmoe
