// Token-to-expert bucketing: histogram, exclusive prefix sum and a stable
// permutation of the routes grouped by expert (PocketLLM design record,
// section 4: the routes are sorted by expert so that every output element has
// exactly one writer and the top-k can be summed in slot order afterwards).
//
// Workgroups of 1024 threads (16 wavefronts), each scattering one block of
// consecutive routes (launch_bucket sizes the blocks: one block for small
// calls); the first workgroup also writes the counts, offsets and chunk
// list.  Integer work only, so the result is bit-exact whatever the
// scheduling.  A block is cut into 16 contiguous segments, one per wavefront,
// in route order:
//   1. each wavefront counts its segment per expert, and the workgroup counts
//      the routes before and after its block per expert (LDS atomics; a count
//      does not depend on order) -- every workgroup reads all the ids;
//   2. per expert, a scan over the 16 segment counts, starting at the routes
//      before the block, gives each wavefront the number of earlier routes of
//      that expert; a scan over the experts gives the expert offsets and the
//      first chunk of each expert;
//   3. each wavefront walks its own segment 64 routes at a time, in order:
//      lanes holding the same expert find each other with one ballot per bit
//      of the expert id and rank themselves by lane; the wavefront's
//      running count per expert carries across steps.  Position = expert
//      offset + earlier blocks and segments + running count + lane rank,
//      which is exactly the stable order (ascending route id in an expert).
// No step after the scans needs a workgroup barrier.
// The same pass writes the work list of the FFN kernels (chunk_rows is a
// power of two), largest chunks first so that the long ones do not start
// last: the shared expert's chunks of chunk_rows tokens, then every full
// chunk of chunk_rows routes of one expert (expert order), then each
// expert's remainder chunk, by size descending (ties by expert index).  The
// order only schedules work: every chunk writes its own outputs.
#include "device.h"
#include "launch.h"

namespace qmoe {

constexpr int kBucketThreads = 1024;
constexpr int kBucketWaves = kBucketThreads / 64;
constexpr int kKeysPerLane = 16;  // routes a lane holds in registers per pass (64 x 16 per wavefront)

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// One step of the scatter: 64 routes in route order (lane = order).  Lanes
// holding the same expert find each other with one ballot per bit of the
// expert id (key_bits of them) and rank themselves by lane; position = expert
// offset + routes of that expert before this step (run, the wavefront's
// running count) + lane rank.  The mask of valid lanes starts the match, so
// the per-bit ballots need no validity term.
__device__ __forceinline__ void scatter_step(bool valid, int key, int r, uint64_t below, int key_bits, int32_t* run,
                                             const int32_t* s_off, int32_t* __restrict__ perm,
                                             int32_t* __restrict__ pos) {
  uint64_t peers = __builtin_amdgcn_ballot_w64(valid);
#pragma unroll
  for (int bit = 0; bit < 8; bit++) {
    if (bit < key_bits) {  // uniform
      const bool set = (key >> bit) & 1;
      const uint64_t b = __builtin_amdgcn_ballot_w64(set);
      peers &= set ? b : ~b;
    }
  }
  const int rank = __popcll(peers & below);
  const int before = run[key];
  if (valid) {
    const int at = s_off[key] + before + rank;
    perm[at] = r;
    if (pos) pos[r] = at;
  }
  __builtin_amdgcn_wave_barrier();
  if (valid && rank == 0) run[key] = before + __popcll(peers);
  __builtin_amdgcn_wave_barrier();
}

__global__ __launch_bounds__(kBucketThreads) void k_bucket(const int32_t* __restrict__ ids, int T, int K, int E,
                                                           int n_shared, int chunk_shift, int block_routes,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ pos, Chunk* __restrict__ chunks,
                                                           int32_t* __restrict__ n_chunks) {
  __shared__ int32_t s_seg[kBucketWaves][256];  // per segment: count, then routes before it, then running
  __shared__ int32_t s_cnt[256];
  __shared__ int32_t s_off[256];
  __shared__ int32_t s_chunk_first[257];
  __shared__ int32_t s_part[3][4];
  __shared__ int32_t s_key[256];  // remainder chunk sort key, or INT32_MAX
  __shared__ int32_t s_before[256], s_after[256];  // routes of each expert before / after this block
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int R = T * K;
  const int b0 = min(R, (int)blockIdx.x * block_routes), b1 = min(R, b0 + block_routes);  // this block
  const int seg = (b1 - b0 + kBucketWaves - 1) / kBucketWaves;
  const int r0 = min(b1, b0 + wave * seg), r1 = min(b1, r0 + seg);
  const bool lead = blockIdx.x == 0;  // writes the counts, offsets and chunk list (every block computes them)

  for (int i = tid; i < kBucketWaves * 256; i += kBucketThreads) (&s_seg[0][0])[i] = 0;
  for (int i = tid; i < 256; i += kBucketThreads) s_before[i] = s_after[i] = 0;
  // the first 64 x kKeysPerLane routes of the segment stay in registers for the scatter
  int key0[kKeysPerLane];
#pragma unroll
  for (int j = 0; j < kKeysPerLane; j++) {
    const int r = r0 + 64 * j + lane;
    key0[j] = r < r1 ? ids[r] : 0;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kKeysPerLane; j++)
    if (r0 + 64 * j + lane < r1) atomicAdd(&s_seg[wave][key0[j]], 1);
  for (int r = r0 + 64 * kKeysPerLane + lane; r < r1; r += 64) atomicAdd(&s_seg[wave][ids[r]], 1);
  for (int r = tid; r < b0; r += kBucketThreads) atomicAdd(&s_before[ids[r]], 1);
  for (int r = b1 + tid; r < R; r += kBucketThreads) atomicAdd(&s_after[ids[r]], 1);
  __syncthreads();

  // per expert: exclusive scan over the segments from the routes before the
  // block, total count, full chunks, remainder
  const int rows = 1 << chunk_shift;
  int cnt = 0, nch = 0, rem = 0;
  if (tid < 256) {
    cnt = s_before[tid];
#pragma unroll
    for (int w = 0; w < kBucketWaves; w++) {
      const int c = s_seg[w][tid];
      s_seg[w][tid] = cnt;
      cnt += c;
    }
    cnt += s_after[tid];
    if (tid >= E) cnt = 0;
    nch = cnt >> chunk_shift;
    rem = cnt & (rows - 1);
    s_cnt[tid] = cnt;
    s_key[tid] = rem > 0 ? ((rows - rem) << 8) | tid : 0x7fffffff;
  }
  // exclusive scan over the experts (four wavefronts of 64 experts)
  int inc_c = 0, inc_n = 0, inc_r = 0;
  if (tid < 256) {
    inc_c = wave_inclusive_scan(cnt, lane);
    inc_n = wave_inclusive_scan(nch, lane);
    inc_r = wave_inclusive_scan(rem > 0 ? 1 : 0, lane);
    if (lane == 63) {
      s_part[0][wave] = inc_c;
      s_part[1][wave] = inc_n;
      s_part[2][wave] = inc_r;
    }
  }
  __syncthreads();
  int n_rem = 0;
  if (tid < 256) {
    int pc = 0, pn = 0;
    for (int w = 0; w < wave; w++) {
      pc += s_part[0][w];
      pn += s_part[1][w];
    }
    s_off[tid] = pc + inc_c - cnt;
    s_chunk_first[tid] = pn + inc_n - nch;
    if (tid == 255) s_chunk_first[256] = pn + inc_n;
  }
  for (int w = 0; w < 4; w++) n_rem += s_part[2][w];
  __syncthreads();
  for (int e = tid; lead && e < E; e += kBucketThreads) {
    counts[e] = s_cnt[e];
    offsets[e] = s_off[e];
  }
  if (lead && tid == 0) offsets[E] = R;

  // chunk list (independent of the permutation itself); optional
  const bool want_chunks = lead && chunks != nullptr;
  const int shared_chunks = n_shared ? (T + rows - 1) >> chunk_shift : 0;
  const int full_chunks = s_chunk_first[256];
  for (int j = tid; want_chunks && j < shared_chunks; j += kBucketThreads) {
    Chunk c;
    c.expert = -1;
    c.first = j << chunk_shift;
    c.count = min(rows, T - (j << chunk_shift));
    c.pad = 0;
    chunks[j] = c;
  }
  if (want_chunks && tid < E) {
    const int c0 = shared_chunks + s_chunk_first[tid];
    for (int j = 0; j < nch; j++) {
      Chunk c;
      c.expert = tid;
      c.first = s_off[tid] + rows * j;
      c.count = rows;
      c.pad = 0;
      chunks[c0 + j] = c;
    }
    if (rem > 0) {
      const int key = s_key[tid];
      int rank = 0;
      for (int q = 0; q < E; q++) rank += s_key[q] < key;
      Chunk c;
      c.expert = tid;
      c.first = s_off[tid] + rows * nch;
      c.count = rem;
      c.pad = 0;
      chunks[shared_chunks + full_chunks + rank] = c;
    }
  }
  if (tid == 0 && want_chunks) *n_chunks = shared_chunks + full_chunks + n_rem;

  // stable scatter, each wavefront over its own segment in route order, 64 x
  // kKeysPerLane routes per pass with all their ids requested at once
  int32_t* run = s_seg[wave];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int key_bits = 0;  // bits of the largest expert id
  while ((1 << key_bits) < E) key_bits++;
  for (int pass = 0; r0 + 64 * kKeysPerLane * pass < r1; pass++) {
    int key_p[kKeysPerLane];
#pragma unroll
    for (int j = 0; j < kKeysPerLane; j++) {
      const int r = r0 + 64 * (kKeysPerLane * pass + j) + lane;
      key_p[j] = pass == 0 ? key0[j] : (r < r1 ? ids[r] : 0);
    }
#pragma unroll
    for (int j = 0; j < kKeysPerLane; j++) {
      const int base = r0 + 64 * (kKeysPerLane * pass + j);
      if (base >= r1) break;
      scatter_step(base + lane < r1, key_p[j], base + lane, below, key_bits, run, s_off, perm, pos);
    }
  }
}

// Blocks of at least kBucketMinBlock routes (one scatter step per wavefront),
// at most kBucketMaxBlocks of them: every workgroup counts all the routes, so
// more blocks only pay while the scatter outweighs that count.
constexpr int kBucketMinBlock = 64 * kBucketWaves;
constexpr int kBucketMaxBlocks = 64;

hipError_t launch_bucket(const int32_t* ids, int T, int K, int E, int n_shared, int chunk_rows, int32_t* counts,
                         int32_t* offsets, int32_t* perm, int32_t* pos, Chunk* chunks, int32_t* n_chunks,
                         hipStream_t stream) {
  int shift = 0;
  while ((1 << shift) < chunk_rows) shift++;
  const int R = T * K;
  int block = (R + kBucketMaxBlocks - 1) / kBucketMaxBlocks;
  block = block < kBucketMinBlock ? kBucketMinBlock : block;
  const int n_blocks = R > 0 ? (R + block - 1) / block : 1;
  clear_last_error();
  hipLaunchKernelGGL(k_bucket, dim3(n_blocks), dim3(kBucketThreads), 0, stream, ids, T, K, E, n_shared, shift, block,
                     counts, offsets, perm, pos, chunks, n_chunks);
  return hipGetLastError();
}

}  // namespace qmoe
