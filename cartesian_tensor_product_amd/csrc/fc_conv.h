// Edge-convolution launch interface shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "fc_common.h"

namespace fc {

struct ConvArgs {
  int N, E, C;
  float rc;
  const int *rowptr, *sender, *receiver, *t_rowptr, *t_edge;
  const float *pos, *shift, *x, *W, *g;
  float *z, *x_bar, *pos_bar, *rbar;
};

#include "generated/fc_conv_configs.h"

bool conv_supported(int l_in, int l_edge, int l_out);
// op 0: forward (needs rowptr, sender, pos, shift, x, W, z);
// op 1: VJP (additionally receiver, t_rowptr, t_edge, g, rbar, and x_bar
//       and/or pos_bar).
void launch_vjp_receiver(const ConvArgs& a, hipStream_t st);
bool conv_dispatch(int op, int l_in, int l_edge, int l_out, const ConvArgs& args, hipStream_t stream);

}  // namespace fc
