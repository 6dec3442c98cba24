// Sender-sorted transpose of the receiver-sorted CSR edge layout.
//
// The FlashCart paper keeps receiver order throughout and accumulates sender
// gradients with atomics (§4 "Comparison with other kernels"); this library
// instead runs its VJP over a sender-sorted copy of the edge list so that
// every output is written once.  The transpose is a counting sort: receiver
// ids per edge, an integer histogram of senders, an exclusive scan, a scatter,
// and a per-sender sort of the scattered edge ids (so the result does not
// depend on the order the scatter's integer atomics were served in).
#include <hip/hip_runtime.h>

#include "fc_graph.h"

namespace fc {

__global__ void graph_receiver_kernel(int N, const int* __restrict__ rowptr, int* __restrict__ receiver,
                                      int* __restrict__ counts) {
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= N) return;
  counts[u] = 0;
  for (int e = rowptr[u]; e < rowptr[u + 1]; ++e) receiver[e] = u;
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
                                     int* __restrict__ t_edge) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) t_edge[atomicAdd(&cursor[sender[e]], 1)] = e;
}

// Insertion sort of each sender's edge ids (segments are short: the
// neighbour count of a node).
__global__ void graph_sort_kernel(int N, const int* __restrict__ t_rowptr, int* __restrict__ t_edge) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= N) return;
  const int lo = t_rowptr[v], hi = t_rowptr[v + 1];
  for (int i = lo + 1; i < hi; ++i) {
    const int key = t_edge[i];
    int j = i - 1;
    while (j >= lo && t_edge[j] > key) {
      t_edge[j + 1] = t_edge[j];
      --j;
    }
    t_edge[j + 1] = key;
  }
}

size_t graph_transpose_ws(int N) { return ((size_t)2 * N * sizeof(int) + 255) / 256 * 256; }

void graph_transpose(int N, int E, const int* rowptr, const int* sender, int* receiver, int* t_rowptr,
                     int* t_edge, void* ws, hipStream_t st) {
  int* counts = static_cast<int*>(ws);
  int* cursor = counts + N;
  const int b = 256;
  hipLaunchKernelGGL(graph_receiver_kernel, dim3((N + b - 1) / b), dim3(b), 0, st, N, rowptr, receiver, counts);
  if (E > 0)
    hipLaunchKernelGGL(graph_hist_kernel, dim3((E + b - 1) / b), dim3(b), 0, st, E, sender, counts);
  hipLaunchKernelGGL(graph_scan_kernel, dim3(1), dim3(1024), 0, st, N, counts, t_rowptr, cursor);
  if (E > 0)
    hipLaunchKernelGGL(graph_scatter_kernel, dim3((E + b - 1) / b), dim3(b), 0, st, E, sender, cursor, t_edge);
  hipLaunchKernelGGL(graph_sort_kernel, dim3((N + b - 1) / b), dim3(b), 0, st, N, t_rowptr, t_edge);
}

}  // namespace fc
