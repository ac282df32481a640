// Capacity and slot assignment: rank every token among the tokens routed to
// its expert under the overflow priority; keep rank < C.
//
// Sources: "MoE expert capacity factor and token dropping" page, After
// overflow and the training-step flowchart (group by expert, count, compare
// with capacity, keep the highest routing weights); "Top-1 Routing" page,
// Token Dropping (tokens beyond the expert buffer skip the expert).
//
// Token order, atomic-free and deterministic:
//   assign_hist  - one workgroup per 256 tokens: each wave finds, for each of
//                  its 64 tokens, the lanes below it with the same expert
//                  (10 ballots over the expert-id bits); per-wave counts meet
//                  in an LDS table, giving each token its rank inside the block
//                  and the block's per-expert histogram.
//   assign_scan  - one workgroup: per-expert exclusive scan of the block
//                  histograms, kept_count = min(total, C), n_dropped, the
//                  ascending list of active experts and segment offsets.
//   assign_slots - slot = block offset + rank in block, kept iff < C; also
//                  marks the empty slots of token_of_slot with -1.
// Gate-descending priority additionally groups each expert's tokens (token
// order) and sorts every group by (gate descending, token ascending) with a
// bitonic sort in LDS (one workgroup per expert); groups larger than the LDS
// tile fall back to counting, for each token, the keys that precede it.
//
// Expert ids outside [0, N) (possible only when a caller feeds its own ids)
// are treated as dropped tokens.
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

constexpr int kAssignBlock = 256;
constexpr int kSegMax = 8192;  // keys per LDS sort (64 KB)

__global__ __launch_bounds__(kAssignBlock) void assign_hist(const int32_t* __restrict__ eid, int64_t T, int N,
                                                            int32_t* __restrict__ blockcount,
                                                            int32_t* __restrict__ local_rank) {
  extern __shared__ int tab[];  // [4][N]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 4 * N; i += kAssignBlock) tab[i] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kAssignBlock + tid;
  int e = (t < T) ? eid[t] : -1;
  const bool valid = e >= 0 && e < N;
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t bm = __ballot(bit);
    same &= bit ? bm : ~bm;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int r = __popcll(same & below);
  if (valid && (same >> lane) == 1ull) tab[w * N + e] = __popcll(same);  // highest lane of its group
  __syncthreads();
  if (t < T) {
    int off = 0;
    if (valid)
      for (int v = 0; v < w; ++v) off += tab[v * N + e];
    local_rank[t] = valid ? off + r : -1;
  }
  for (int n = tid; n < N; n += kAssignBlock)
    blockcount[(int64_t)blockIdx.x * N + n] = tab[n] + tab[N + n] + tab[2 * N + n] + tab[3 * N + n];
}

__global__ __launch_bounds__(1024) void assign_scan(const int32_t* __restrict__ blockcount, int64_t nblk, int64_t T,
                                                    int N, int C, int32_t* __restrict__ blockoff,
                                                    int32_t* __restrict__ total, int32_t* __restrict__ kept_count,
                                                    int32_t* __restrict__ n_dropped, int32_t* __restrict__ active,
                                                    int32_t* __restrict__ n_active,
                                                    int32_t* __restrict__ seg_start) {
  __shared__ int wsum[16];
  const int n = threadIdx.x;
  int run = 0, kept = 0;
  if (n < N) {
    int64_t b = 0;
    for (; b + 8 <= nblk; b += 8) {  // 8 loads in flight, then the running sum
      int cv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) cv[u] = blockcount[(b + u) * N + n];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        blockoff[(b + u) * N + n] = run;
        run += cv[u];
      }
    }
    for (; b < nblk; ++b) {
      const int c = blockcount[b * N + n];
      blockoff[b * N + n] = run;
      run += c;
    }
    total[n] = run;
    kept = run < C ? run : C;
    kept_count[n] = kept;
  }
  int tot_kept, tot_active, tot_routed;
  const int seg = block_exclusive_scan(n < N ? run : 0, wsum, &tot_routed);
  const int pos = block_exclusive_scan(kept > 0 ? 1 : 0, wsum, &tot_active);
  block_exclusive_scan(kept, wsum, &tot_kept);
  if (n < N) {
    seg_start[n] = seg;
    if (kept > 0) active[pos] = n;
  }
  if (n == 0) {
    n_active[0] = tot_active;
    n_dropped[0] = (int32_t)(T - tot_kept);
  }
}

__global__ __launch_bounds__(kAssignBlock) void assign_slots(const int32_t* __restrict__ eid,
                                                             const int32_t* __restrict__ local_rank,
                                                             const int32_t* __restrict__ blockoff,
                                                             const int32_t* __restrict__ kept_count, int64_t T, int N,
                                                             int C, int32_t* __restrict__ slot,
                                                             int32_t* __restrict__ token_of_slot) {
  const int64_t i = (int64_t)blockIdx.x * kAssignBlock + threadIdx.x;
  if (i < T) {
    const int e = eid[i];
    int s = -1;
    if (e >= 0 && e < N) {
      const int r = blockoff[(i / kAssignBlock) * N + e] + local_rank[i];
      if (r < C) {
        s = r;
        token_of_slot[(int64_t)e * C + r] = (int32_t)i;
      }
    }
    slot[i] = s;
  }
  if (i < (int64_t)N * C) {
    const int e = (int)(i / C), s = (int)(i - (int64_t)e * C);
    if (s >= kept_count[e]) token_of_slot[i] = -1;
  }
}

// token-order grouping of every expert's tokens (no capacity cut)
__global__ __launch_bounds__(kAssignBlock) void assign_group(const int32_t* __restrict__ eid,
                                                             const int32_t* __restrict__ local_rank,
                                                             const int32_t* __restrict__ blockoff,
                                                             const int32_t* __restrict__ seg_start, int64_t T, int N,
                                                             int32_t* __restrict__ perm, int32_t* __restrict__ slot) {
  const int64_t i = (int64_t)blockIdx.x * kAssignBlock + threadIdx.x;
  if (i >= T) return;
  const int e = eid[i];
  if (e >= 0 && e < N)
    perm[seg_start[e] + blockoff[(i / kAssignBlock) * N + e] + local_rank[i]] = (int32_t)i;
  else
    slot[i] = -1;
}

__device__ __forceinline__ uint64_t gate_key(const float* gate, int32_t t) {
  // ascending key == descending gate, then ascending token (gates are > 0)
  return ((uint64_t)(~__float_as_uint(gate[t])) << 32) | (uint32_t)t;
}

__global__ __launch_bounds__(1024) void assign_sort_gate(const int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ seg_start,
                                                         const int32_t* __restrict__ total,
                                                         const float* __restrict__ gate, int N, int C,
                                                         int32_t* __restrict__ slot,
                                                         int32_t* __restrict__ token_of_slot,
                                                         uint64_t* __restrict__ gkeys) {
  extern __shared__ uint64_t keys[];  // kSegMax
  __shared__ int hist[256];
  __shared__ int sel[2];
  __shared__ uint64_t kept_keys[1024];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int n = total[e], base = seg_start[e];
  const int kept = n < C ? n : C;
  for (int s = kept + tid; s < C; s += 1024) token_of_slot[(int64_t)e * C + s] = -1;
  if (n == 0) return;
  if (n <= kSegMax && kept <= 1024) {
    // Only the `kept` smallest keys get slots.  Find the kept-th smallest key
    // by a radix select (8 passes of 8-bit digits, histograms in LDS), gather
    // the keys at or below it, and rank each by counting the smaller ones
    // (keys are unique, so the result does not depend on the gather order).
    for (int i = tid; i < n; i += 1024) keys[i] = gate_key(gate, perm[base + i]);
    uint64_t prefix = 0, mask = 0;
    int want = kept;  // 1-based rank of the threshold among the keys matching prefix
    if (kept < n) {
      for (int shift = 56; shift >= 0; shift -= 8) {
        for (int b = tid; b < 256; b += 1024) hist[b] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += 1024) {
          const uint64_t k = keys[i];
          if ((k & mask) == prefix) atomicAdd(&hist[(int)((k >> shift) & 255)], 1);
        }
        __syncthreads();
        if (tid < 64) {  // one wave: 4 bins per lane, ascending digit order
          int h[4], sum = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            h[q] = hist[tid * 4 + q];
            sum += h[q];
          }
          int incl = sum;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(incl, o, 64);
            if (tid >= o) incl += u;
          }
          int below = incl - sum;  // count in digits < 4 * tid
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (below < want && want <= below + h[q]) {
              sel[0] = tid * 4 + q;
              sel[1] = below;
            }
            below += h[q];
          }
        }
        __syncthreads();
        const int d = sel[0];
        want -= sel[1];
        prefix |= (uint64_t)d << shift;
        mask |= (uint64_t)255 << shift;
        __syncthreads();  // sel and hist are rewritten in the next pass
      }
    } else {
      prefix = ~0ull;  // every key is kept
    }
    if (tid == 0) sel[0] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 1024) {
      const uint64_t k = keys[i];
      if (k <= prefix) kept_keys[atomicAdd(&sel[0], 1)] = k;
      else slot[(int32_t)(k & 0xffffffffull)] = -1;
    }
    __syncthreads();
    if (tid < kept) {
      const uint64_t own = kept_keys[tid];
      int r = 0;
      for (int j = 0; j < kept; ++j) r += kept_keys[j] < own ? 1 : 0;
      const int32_t t = (int32_t)(own & 0xffffffffull);
      slot[t] = r;
      token_of_slot[(int64_t)e * C + r] = t;
    }
    return;
  }
  if (n <= kSegMax) {
    int P = 1;
    while (P < n) P <<= 1;
    for (int i = tid; i < P; i += 1024) keys[i] = (i < n) ? gate_key(gate, perm[base + i]) : ~0ull;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P; i += 1024) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint64_t a = keys[i], b = keys[ixj];
            const bool up = (i & k) == 0;
            if ((a > b) == up) {
              keys[i] = b;
              keys[ixj] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < n; i += 1024) {
      const int32_t t = (int32_t)(keys[i] & 0xffffffffull);
      if (i < C) {
        slot[t] = i;
        token_of_slot[(int64_t)e * C + i] = t;
      } else {
        slot[t] = -1;
      }
    }
    return;
  }
  // large group: rank = number of keys below one's own, counted over LDS tiles
  for (int i = tid; i < n; i += 1024) gkeys[base + i] = gate_key(gate, perm[base + i]);
  __threadfence();
  __syncthreads();
  for (int c0 = 0; c0 < n; c0 += 1024) {
    const int i = c0 + tid;
    const bool mine = i < n;
    const uint64_t own = mine ? gkeys[base + i] : ~0ull;
    int cnt = 0;
    for (int tile = 0; tile < n; tile += kSegMax) {
      const int len = (n - tile) < kSegMax ? (n - tile) : kSegMax;
      for (int j = tid; j < len; j += 1024) keys[j] = gkeys[base + tile + j];
      __syncthreads();
      for (int j = 0; j < len; ++j) cnt += keys[j] < own ? 1 : 0;
      const bool done = __syncthreads_and(!mine || cnt >= C);
      if (done) break;
    }
    if (mine) {
      const int32_t t = (int32_t)(own & 0xffffffffull);
      if (cnt < C) {
        slot[t] = cnt;
        token_of_slot[(int64_t)e * C + cnt] = t;
      } else {
        slot[t] = -1;
      }
    }
  }
}

// ----------------------------------------------------------------------------
AssignPlan assign_plan(int64_t T, int N, int C, int priority) {
  (void)C;
  AssignPlan pl{};
  pl.nblk = (T + kAssignBlock - 1) / kAssignBlock;
  size_t off = 0;
  pl.off_blockcount = off;
  off = align_up(off + (size_t)pl.nblk * N * 4);
  pl.off_blockoff = off;
  off = align_up(off + (size_t)pl.nblk * N * 4);
  pl.off_local_rank = off;
  off = align_up(off + (size_t)T * 4);
  pl.off_total = off;
  off = align_up(off + (size_t)N * 4);
  pl.off_seg_start = off;
  off = align_up(off + (size_t)N * 4);
  pl.off_perm = off;
  pl.off_keys = off;
  if (priority == 1) {
    off = align_up(off + (size_t)T * 4);
    pl.off_keys = off;
    off = align_up(off + (size_t)T * 8);
  }
  pl.bytes = off;
  return pl;
}

hipError_t launch_assign(const AssignPlan& pl, const int32_t* expert_id, const float* gate, int64_t T, int N, int C,
                         int priority, int32_t* slot, int32_t* token_of_slot, int32_t* kept_count,
                         int32_t* n_dropped, int32_t* active, int32_t* n_active, char* ws, hipStream_t st) {
  int32_t* blockcount = reinterpret_cast<int32_t*>(ws + pl.off_blockcount);
  int32_t* blockoff = reinterpret_cast<int32_t*>(ws + pl.off_blockoff);
  int32_t* local_rank = reinterpret_cast<int32_t*>(ws + pl.off_local_rank);
  int32_t* total = reinterpret_cast<int32_t*>(ws + pl.off_total);
  int32_t* seg_start = reinterpret_cast<int32_t*>(ws + pl.off_seg_start);
  hipLaunchKernelGGL(assign_hist, dim3((unsigned)pl.nblk), dim3(kAssignBlock), (size_t)4 * N * 4, st, expert_id, T, N,
                     blockcount, local_rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(assign_scan, dim3(1), dim3(1024), 0, st, blockcount, pl.nblk, T, N, C, blockoff, total,
                     kept_count, n_dropped, active, n_active, seg_start);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (priority == 0) {
    const int64_t cnt = T > (int64_t)N * C ? T : (int64_t)N * C;
    hipLaunchKernelGGL(assign_slots, dim3((unsigned)((cnt + kAssignBlock - 1) / kAssignBlock)), dim3(kAssignBlock), 0,
                       st, expert_id, local_rank, blockoff, kept_count, T, N, C, slot, token_of_slot);
    return hipGetLastError();
  }
  int32_t* perm = reinterpret_cast<int32_t*>(ws + pl.off_perm);
  uint64_t* gkeys = reinterpret_cast<uint64_t*>(ws + pl.off_keys);
  hipLaunchKernelGGL(assign_group, dim3((unsigned)pl.nblk), dim3(kAssignBlock), 0, st, expert_id, local_rank, blockoff,
                     seg_start, T, N, perm, slot);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(assign_sort_gate, dim3((unsigned)N), dim3(1024), (size_t)kSegMax * 8, st, perm, seg_start, total,
                     gate, N, C, slot, token_of_slot, gkeys);
  return hipGetLastError();
}

}  // namespace swm
