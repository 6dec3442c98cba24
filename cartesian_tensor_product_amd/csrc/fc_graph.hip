// Sender-sorted transpose of the receiver-sorted CSR edge layout.
//
// The FlashCart paper keeps receiver order throughout and accumulates sender
// gradients with atomics (§4 "Comparison with other kernels"); this library
// instead runs its VJP over a sender-sorted copy of the edge list so that
// every output is written once.  The transpose is a counting sort:
//   1. an integer histogram of senders (the counts do not depend on the
//      order in which the integer atomics are served);
//   2. an exclusive scan into t_rowptr;
//   3. a scatter of the edge ids into their sender's segment, in arrival
//      order, staged in `receiver` (which is written last);
//   4. one wave per sender ranks the ids of its segment: the ids are
//      distinct, so an id's position is the number of smaller ids in the
//      segment, and the segment comes out in ascending order whatever the
//      scatter's order was;
//   5. receiver[e] = u, one wave per receiver.
// Step 4 costs O(n^2 / 64) comparisons per wave for a segment of n ids.
#include <hip/hip_runtime.h>

#include <climits>

#include "fc_graph.h"

namespace fc {

namespace {
constexpr int kGraphWaves = 4;   // waves per block in the per-node kernels
}

__global__ void graph_zero_kernel(int N, int* __restrict__ counts) {
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u < N) counts[u] = 0;
}

__global__ void graph_hist_kernel(int E, const int* __restrict__ sender, int* __restrict__ counts) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) atomicAdd(&counts[sender[e]], 1);
}

// Exclusive scan by a single block: each thread sums a contiguous slice,
// the block scans the slice totals, then each thread writes its slice.
__global__ __launch_bounds__(1024) void graph_scan_kernel(int N, const int* __restrict__ counts,
                                                         int* __restrict__ t_rowptr,
                                                         int* __restrict__ cursor) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int lo = min(N, t * per), hi = min(N, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += counts[i];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - s;
  for (int i = lo; i < hi; ++i) {
    t_rowptr[i] = run;
    cursor[i] = run;
    run += counts[i];
  }
  if (t == 1023) t_rowptr[N] = part[1023];
}

__global__ void graph_scatter_kernel(int E, const int* __restrict__ sender, int* __restrict__ cursor,
                                     int* __restrict__ staged) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) staged[atomicAdd(&cursor[sender[e]], 1)] = e;
}

// One wave per sender v: lane i takes ids i, i + 64, ... of the segment and
// counts the smaller ids of the whole segment, read 64 at a time and
// broadcast lane by lane.
__global__ __launch_bounds__(kGraphWaves * 64) void graph_rank_kernel(int N, const int* __restrict__ t_rowptr,
                                                                    const int* __restrict__ staged,
                                                                    int* __restrict__ t_edge) {
  const int lane = threadIdx.x % 64;
  const int v = blockIdx.x * kGraphWaves + threadIdx.x / 64;
  if (v >= N) return;
  const int lo = t_rowptr[v], n = t_rowptr[v + 1] - lo;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const int key = i < n ? staged[lo + i] : INT_MAX;
    int rank = 0;
    for (int j0 = 0; j0 < n; j0 += 64) {
      const int kj = j0 + lane < n ? staged[lo + j0 + lane] : INT_MAX;
      const int m = min(64, n - j0);
      if (m == 64) {
#pragma unroll
        for (int t = 0; t < 64; ++t) rank += __builtin_amdgcn_readlane(kj, t) < key;
      } else {
        for (int t = 0; t < m; ++t) rank += __builtin_amdgcn_readlane(kj, t) < key;
      }
    }
    if (i < n) t_edge[lo + rank] = key;
  }
}

__global__ __launch_bounds__(kGraphWaves * 64) void graph_receiver_kernel(int N, const int* __restrict__ rowptr,
                                                                        int* __restrict__ receiver) {
  const int lane = threadIdx.x % 64;
  const int u = blockIdx.x * kGraphWaves + threadIdx.x / 64;
  if (u >= N) return;
  const int e1 = rowptr[u + 1];
  for (int e = rowptr[u] + lane; e < e1; e += 64) receiver[e] = u;
}

size_t graph_transpose_ws(int N) { return ((size_t)2 * N * sizeof(int) + 255) / 256 * 256; }

void graph_transpose(int N, int E, const int* rowptr, const int* sender, int* receiver, int* t_rowptr,
                     int* t_edge, void* ws, hipStream_t st) {
  int* counts = static_cast<int*>(ws);
  int* cursor = counts + N;
  const int b = 256;
  const dim3 per_node((N + kGraphWaves - 1) / kGraphWaves), wave_block(kGraphWaves * 64);
  hipLaunchKernelGGL(graph_zero_kernel, dim3((N + b - 1) / b), dim3(b), 0, st, N, counts);
  if (E > 0)
    hipLaunchKernelGGL(graph_hist_kernel, dim3((E + b - 1) / b), dim3(b), 0, st, E, sender, counts);
  hipLaunchKernelGGL(graph_scan_kernel, dim3(1), dim3(1024), 0, st, N, counts, t_rowptr, cursor);
  if (E > 0) {
    hipLaunchKernelGGL(graph_scatter_kernel, dim3((E + b - 1) / b), dim3(b), 0, st, E, sender, cursor, receiver);
    hipLaunchKernelGGL(graph_rank_kernel, per_node, wave_block, 0, st, N, t_rowptr, receiver, t_edge);
    hipLaunchKernelGGL(graph_receiver_kernel, per_node, wave_block, 0, st, N, rowptr, receiver);
  }
}

}  // namespace fc
