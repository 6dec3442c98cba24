// Sender-sorted transpose of a receiver-sorted CSR graph.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace fc {

size_t graph_transpose_ws(int N);
void graph_transpose(int N, int E, const int* rowptr, const int* sender, int* receiver, int* t_rowptr,
                     int* t_edge, void* ws, hipStream_t st);

}  // namespace fc
