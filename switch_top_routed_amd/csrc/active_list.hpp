// The token-order assignment's cross-expert results built inside the first
// expert GEMM (shared by the bf16 and MXFP4 streaming GEMMs).
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

// Every workgroup of the first GEMM builds the active list from the kept
// counts (thread i takes experts 4i .. 4i + 3, so a block scan keeps expert
// order); workgroup 0 also writes the list, n_active, n_dropped and L_aux.
// Returns n_active; the list is left in s_act.
template <int NTH>
__device__ int active_from_kept(const ActiveFromKept& afk, int N, int* s_act, int* wsum, double* sl) {
  constexpr int PER = 1024 / NTH;  // N <= 1024
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int kv[PER], cnt = 0, ksum = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int n = tid * PER + q;
    kv[q] = n < N ? afk.kept[n] : 0;
    cnt += kv[q] > 0 ? 1 : 0;
    ksum += kv[q];
  }
  int n_act, kept_tot;
  int pos = block_exclusive_scan(cnt, wsum, &n_act);
  block_exclusive_scan(ksum, wsum, &kept_tot);
#pragma unroll
  for (int q = 0; q < PER; ++q)
    if (kv[q] > 0) s_act[pos++] = tid * PER + q;
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int a = tid; a < n_act; a += NTH) afk.active[a] = s_act[a];
    // L_aux through route_finalize's tree: 16 groups of 64 experts, an xor tree
    // inside each group, then the group sums in group order
    for (int g = w; g < 16; g += NTH / 64) {
      const int n = g * 64 + lane;
      double t = n < N ? afk.term[n] : 0.0;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
      if (lane == 0) sl[g] = t;
    }
    __syncthreads();
    if (tid == 0) {
      double a = 0.0;
      for (int i = 0; i < 16; ++i) a += sl[i];
      afk.l_aux[0] = (float)((double)N * a);
      afk.n_active[0] = n_act;
      afk.n_dropped[0] = (int32_t)(afk.TV - kept_tot);
    }
  }
  return n_act;
}

}  // namespace swm
