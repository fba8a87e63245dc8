// Grouping the (token, slot) pairs by expert: per-chunk histograms, one scan over
// (chunk x expert), a stable scatter, and an optional coalesced row gather.
//
// Transformers "Experts backends" page, backends table row grouped_mm: tokens are sorted by their
// selected expert so one grouped GEMM projects them all. The order inside an expert is the flat
// pair index (stable), which makes the permutation deterministic.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kChunk = 1024;       // pairs per block in the histogram and scatter kernels
constexpr int kScatterThreads = 256;

// An expert id outside [0, E) is a caller error. Such a pair is left out of every count, its
// pair_pos entry is set to -1 and offsets[E] becomes the number of in-range pairs, so the error
// shows as offsets[E] < P and no LDS or global address is formed from the bad id.
__device__ __forceinline__ bool in_range(int e, int E) {
  return static_cast<unsigned>(e) < static_cast<unsigned>(E);
}

__global__ __launch_bounds__(256) void chunk_histogram_kernel(const int32_t* __restrict__ ids,
                                                              int P, int E,
                                                              int32_t* __restrict__ chunk_hist) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kChunk;
  const int p1 = min(P, p0 + kChunk);
  for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int e = ids[p];
    if (in_range(e, E)) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    chunk_hist[static_cast<size_t>(blockIdx.x) * E + e] = hist[e];
}

// Walks expert e's chunk counts over chunks [c0, c1), adding them to run (and, with kBase, writing
// each chunk's starting position first). Counts are loaded in batches whose loads all issue before
// any is used (a loop adding each count as it arrives waits a full memory round trip per chunk):
// 16 at a time while more than 8 remain, then 4, then one, so short ranges load little extra.
// Batch slots past c1 reread chunk c1 - 1 and are not used.
template <int B, bool kBase>
__device__ __forceinline__ void chunk_batch(const int32_t* __restrict__ chunk_hist, int cb, int c1,
                                            int E, int e, int& run,
                                            int32_t* __restrict__ chunk_base) {
  int v[B];
#pragma unroll
  for (int u = 0; u < B; ++u) v[u] = chunk_hist[static_cast<size_t>(min(cb + u, c1 - 1)) * E + e];
#pragma unroll
  for (int u = 0; u < B; ++u) {
    if (cb + u < c1) {
      if constexpr (kBase) chunk_base[static_cast<size_t>(cb + u) * E + e] = run;
      run += v[u];
    }
  }
}
template <bool kBase>
__device__ __forceinline__ void chunk_walk(const int32_t* __restrict__ chunk_hist, int c0, int c1,
                                           int E, int e, int& run,
                                           int32_t* __restrict__ chunk_base) {
  int cb = c0;
  for (; c1 - cb > 8; cb += 16) chunk_batch<16, kBase>(chunk_hist, cb, c1, E, e, run, chunk_base);
  for (; c1 - cb > 1; cb += 4) chunk_batch<4, kBase>(chunk_hist, cb, c1, E, e, run, chunk_base);
  if (cb < c1) chunk_batch<1, kBase>(chunk_hist, cb, c1, E, e, run, chunk_base);
}

// One block of 1024 threads. counts[e] = sum over chunks; offsets = exclusive scan over experts;
// chunk_base[c][e] = offsets[e] + pairs of expert e in chunks before c. Thread (part, e) with
// tid = part * EP + e (EP = E rounded up to a power of two) owns a contiguous range of the chunks
// of expert e, so the G = 1024 / EP parts read the histogram side by side.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ chunk_hist,
                                                    int nchunks, int E, int EP, int P,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ chunk_base) {
  __shared__ int part_sum[kMaxExperts];
  __shared__ int s[kMaxExperts];
  const int tid = threadIdx.x;
  const int G = kMaxExperts / EP;
  const int part = tid / EP, e = tid % EP;
  const int c0 = static_cast<int>(static_cast<long>(part) * nchunks / G);
  const int c1 = static_cast<int>(static_cast<long>(part + 1) * nchunks / G);
  int sum = 0;
  if (e < E) chunk_walk<false>(chunk_hist, c0, c1, E, e, sum, nullptr);
  part_sum[tid] = sum;
  __syncthreads();
  // per expert: total over parts, and each part's exclusive prefix (kept in part_sum)
  int total = 0;
  if (tid < EP) {
    for (int q = 0; q < G; ++q) {
      const int v = part_sum[q * EP + tid];
      part_sum[q * EP + tid] = total;
      total += v;
    }
    if (tid < E) counts[tid] = total;
  }
  s[tid] = total;
  __syncthreads();
  // Hillis-Steele inclusive scan over the experts' totals (the first EP entries; the rest are 0).
  for (int o = 1; o < EP; o <<= 1) {
    int v = (tid >= o) ? s[tid - o] : 0;
    __syncthreads();
    s[tid] += v;
    __syncthreads();
  }
  if (e < E) {
    // start of expert e (inclusive scan of the experts before it) + this part's prefix
    int run = (e > 0 ? s[e - 1] : 0) + part_sum[tid];
    if (part == 0) offsets[e] = run;
    chunk_walk<true>(chunk_hist, c0, c1, E, e, run, chunk_base);
  }
  if (tid == 0) offsets[E] = s[EP - 1];
}

// Stable scatter of pairs [p0, p1) given each expert's next position in `cursor` (LDS). Pairs
// are taken 256 at a time in flat order; inside a wave, lanes holding the same expert are found
// with one ballot per expert-id bit, and a lane's rank is the number of such lanes below it. The
// four waves then claim their positions one after another from the running per-expert cursor, so
// positions follow the flat pair order exactly. Called by all 256 threads of the block.
__device__ __forceinline__ void scatter_range(const int32_t* __restrict__ ids, int p0, int p1,
                                              int E, int id_bits, int* cursor,
                                              int32_t* __restrict__ sorted_pair,
                                              int32_t* __restrict__ pair_pos) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = p0; base < p1; base += kScatterThreads) {
    const int p = base + threadIdx.x;
    const int raw = p < p1 ? ids[p] : 0;
    const bool valid = p < p1 && in_range(raw, E);
    const int e = valid ? raw : 0;
    if (p < p1 && !valid) pair_pos[p] = -1;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(bit);
      match &= bit ? ones : ~ones;
    }
    const int rank = __popcll(match & below);
    const int cnt = __popcll(match);
    for (int w = 0; w < kScatterThreads / kWave; ++w) {
      if (w == wave && valid) {
        const int pos = cursor[e] + rank;
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
        if (rank == 0) cursor[e] = pos + cnt;
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kScatterThreads) void scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, int id_bits,
    const int32_t* __restrict__ chunk_base, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos) {
  __shared__ int cursor[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    cursor[e] = chunk_base[static_cast<size_t>(blockIdx.x) * E + e];
  __syncthreads();
  scatter_range(ids, blockIdx.x * kChunk, min(P, (blockIdx.x + 1) * kChunk), E, id_bits, cursor,
                sorted_pair, pair_pos);
}

// All of the above in one workgroup when the pairs fit in one chunk (P <= kChunk, e.g. decode):
// histogram, exclusive scan over the experts, stable scatter.
__global__ __launch_bounds__(kScatterThreads) void permute_small_kernel(
    const int32_t* __restrict__ ids, int P, int E, int id_bits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos) {
  __shared__ int cursor[kMaxExperts];
  __shared__ int part[kScatterThreads];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kScatterThreads) cursor[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kScatterThreads) {
    const int e = ids[p];
    if (in_range(e, E)) atomicAdd(&cursor[e], 1);
  }
  __syncthreads();
  // thread t scans experts [t per, (t + 1) per); a block scan of the 256 partial sums gives each
  // run's start
  const int per = (E + kScatterThreads - 1) / kScatterThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int sum = 0;
  for (int e = e0; e < e1; ++e) sum += cursor[e];
  part[tid] = sum;
  __syncthreads();
  // scan the first NP partial sums (NP: a power of two covering the threads that hold experts;
  // the others hold 0)
  const int nparts = (E + per - 1) / per;
  int NP = 1;
  while (NP < nparts) NP <<= 1;
  for (int o = 1; o < NP; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int e = e0; e < e1; ++e) {
    const int c = cursor[e];
    counts[e] = c;
    offsets[e] = run;
    cursor[e] = run;
    run += c;
  }
  if (tid == 0) offsets[E] = part[NP - 1];
  __syncthreads();
  scatter_range(ids, 0, P, E, id_bits, cursor, sorted_pair, pair_pos);
}

// x_perm[r] = x[sorted_pair[r] / k]; one wave per row, 16-byte vectors when the row allows it.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ x,
                                                          size_t row_bytes,
                                                          const int32_t* __restrict__ sorted_pair,
                                                          int P, int k,
                                                          uint8_t* __restrict__ x_perm) {
  const int r = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (r >= P) return;
  const int pair = sorted_pair[r];
  if (static_cast<unsigned>(pair) >= static_cast<unsigned>(P)) return;  // a row left unwritten
  const int t = pair / k;
  const uint8_t* src = x + static_cast<size_t>(t) * row_bytes;
  uint8_t* dst = x_perm + static_cast<size_t>(r) * row_bytes;
  const int lane = lane_id();
  if ((row_bytes & 15) == 0 && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(x_perm)) & 15) == 0) {
    const size_t n = row_bytes / 16;
    for (size_t i = lane; i < n; i += kWave)
      reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  } else {
    for (size_t i = lane; i < row_bytes; i += kWave) dst[i] = src[i];
  }
}

}  // namespace

size_t permute_workspace_bytes(int P, int E) {
  const size_t nchunks = (static_cast<size_t>(P) + kChunk - 1) / kChunk;
  return 2 * nchunks * static_cast<size_t>(E) * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, void* workspace,
                          hipStream_t stream) {
  const int nchunks = (P + kChunk - 1) / kChunk;
  int32_t* chunk_hist = static_cast<int32_t*>(workspace);
  int32_t* chunk_base = chunk_hist + static_cast<size_t>(nchunks) * E;
  int id_bits = 0;
  while ((1 << id_bits) < E) ++id_bits;
  if (nchunks == 1) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kScatterThreads), 0, stream, ids, P, E,
                       id_bits, counts, offsets, sorted_pair, pair_pos);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(chunk_histogram_kernel, dim3(nchunks), dim3(256), 0, stream, ids, P, E,
                     chunk_hist);
  int EP = 1;
  while (EP < E) EP <<= 1;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kMaxExperts), 0, stream, chunk_hist, nchunks, E, EP,
                     P, counts, offsets, chunk_base);
  hipLaunchKernelGGL(scatter_kernel, dim3(nchunks), dim3(kScatterThreads), 0, stream, ids, P, E,
                     id_bits, chunk_base, sorted_pair, pair_pos);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, size_t row_bytes, const int32_t* sorted_pair, int P,
                              int k, void* x_perm, hipStream_t stream) {
  dim3 grid((P + 3) / 4), block(256);
  hipLaunchKernelGGL(gather_rows_kernel, grid, block, 0, stream, static_cast<const uint8_t*>(x),
                     row_bytes, sorted_pair, P, k, static_cast<uint8_t*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
