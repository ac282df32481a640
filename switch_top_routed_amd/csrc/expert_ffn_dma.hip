// Expert FFN for large per-expert row counts, weights staged by direct
// global-to-LDS loads.
//
// Same operation as the weight-streaming kernel (out = act(A . W) over the
// filled slots of the active experts; "Top-1 Routing" page, Key parameters and
// compute), for experts with more than 64 rows and for the always-on shared
// dense expert, where the work per weight byte is high enough that MFMA
// throughput and panel reuse matter.  A workgroup (2 x 2 waves, or 2 x 4 for
// the widest tiles) owns a BM x TN output tile and walks K in 32-deep steps:
//  * every global load is a buffer load that writes LDS directly (16 bytes per
//    lane, 1 KB per wave instruction), so the operands never pass through
//    registers on their way in and S LDS stages (separate LDS arrays) keep
//    S - 1 steps of loads in flight with no register ring;
//  * the weight block stays in LDS as it is in memory (k-rows, columns
//    contiguous); the MFMA B fragments (8 consecutive k of one column per lane)
//    come from two ds_read_b64_tr_b16 transposing reads, which need no register
//    transposes.  Within a group of 16 lanes that instruction hands lane i the
//    element i % 4 of the 4-element rows addressed by lanes 4q + i / 4, q = 0..3;
//    so lanes 4q + p point at k-row q, columns 4p .. 4p + 3 of the fragment;
//  * one workgroup barrier per step, without the memory fence that would make
//    every wave wait for all of its in-flight loads: each wave waits for its
//    own loads of the step (vmcnt), then the barrier publishes them.
// A 16-byte chunks are XOR-swizzled by row with two parity bits (bit 0 =
// r1 ^ r2, bit 1 = r1 ^ r3 ^ r6), which keeps the 16-byte fragment reads free
// of bank conflicts for 8- and 16-lane LDS service; weight chunks are XORed
// with 2 (k mod 4) + 8 (k / 8 mod 2), which puts the 8 k-rows that one
// transposing read touches (4 per 16-lane group) on distinct banks.  Two
// waves share each SIMD (two 4-wave workgroups per CU, or one of 8 waves), so
// one wave's MFMAs overlap the other's LDS reads and barrier; tiles are dealt
// to the 8 XCDs in contiguous
// ranges, up to 8 m-chunks of an expert walking the column blocks together
// (shared A and W panels in L2).
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

namespace {

constexpr int kDmaXcds = 8;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// A tile: 16-byte chunk q of row r at r * 64 + ((q ^ swz(r)) << 4)
__device__ __forceinline__ int a_swz(int r) {
  return (((r >> 1) ^ (r >> 2)) & 1) | ((((r >> 1) ^ (r >> 3) ^ (r >> 6)) & 1) << 1);
}
// W tile: 16-byte chunk c of k-row k at k * row_bytes + ((c ^ w_swz(k)) << 4)
__device__ __forceinline__ int w_swz(int k) { return 2 * ((k & 3) | ((k >> 1) & 4)); }

// s_waitcnt vmcnt(n) lgkmcnt(0), expcnt untouched (gfx9 encoding)
#define SWM_WAIT_VMCNT_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// The gfx950 builtins sit in plain (non-template) functions: inside a kernel
// template the host compilation pass rejects them as a substitution failure
// and silently drops the kernel's launch stub.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}
// the same with the non-temporal cache policy (bytes read once per launch)
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 2);
}
__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* lds) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)lds));
}

// y piece (8 bf16) of token t at column col from the S piece sv: the same
// arithmetic, in the same order, as combine_rows (dispatch_combine.hip), so the
// fused layer is bit-identical to the separate combine
__device__ __forceinline__ void combine_piece(const CombineArgs& cb, const u32x4& sv, int64_t t, int col, int d) {
  const int s = cb.slot[t];
  const int e = s >= 0 ? cb.expert_id[t] : 0;
  const bool kept = s >= 0 && s < cb.C && e >= 0 && e < cb.N;
  const float scale = (cb.flags & SWITCH_GATE_SCALE) ? cb.gate[t] : 1.0f;
  const bool res = (cb.flags & SWITCH_RESIDUAL_ALL) != 0;
  const bool need_x = !kept || res;
  const u32x4 xv = need_x ? *reinterpret_cast<const u32x4*>(cb.x + t * d + col) : u32x4{0u, 0u, 0u, 0u};
  const u32x4 ov = kept ? *reinterpret_cast<const u32x4*>(cb.eo + ((int64_t)e * cb.C + s) * d + col)
                        : u32x4{0u, 0u, 0u, 0u};
  float v[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = bf2f(xv[q] & 0xffffu);
    v[2 * q + 1] = bf2f(xv[q] >> 16);
  }
  if (kept) {
    float o[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[2 * q] = bf2f(ov[q] & 0xffffu);
      o[2 * q + 1] = bf2f(ov[q] >> 16);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = res ? v[q] + scale * o[q] : scale * o[q];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] += bf2f(sv[q] & 0xffffu);
    v[2 * q + 1] += bf2f(sv[q] >> 16);
  }
  u32x4 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) out[q] = pack_bf2(v[2 * q], v[2 * q + 1]);
  __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(cb.y + t * d + col));
}

}  // namespace

// MTW m-tiles x NJ n-tiles of 16 x 16 per wave (2 x WN waves): a BM = 32 MTW
// by TN = 16 NJ WN tile; S LDS stages.  WNT: the weights are read once per
// launch (one m-chunk per expert), so their loads carry the non-temporal policy
// and leave the caches to the token rows, which every column block re-reads.
// CMB: the dense (shared-expert) second GEMM also does the top-1 combine
// (CombineArgs): each 16-byte piece of S becomes the piece of y.
template <int MTW, int NJ, int S, bool WNT, int WN, bool CMB>
__global__ __launch_bounds__(128 * WN, WN > 2 || MTW * NJ >= 48 ? 1 : 2) void ffn_tile_dma(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, uint16_t* __restrict__ out,
    const int32_t* __restrict__ kept_count, const int32_t* __restrict__ active, const int32_t* __restrict__ n_active,
    int N, int C, int K, int Ncols, int relu, int mch, const int32_t* __restrict__ gather, int64_t a_rows,
    CombineArgs cmb) {
  constexpr int NWV = 2 * WN;          // waves
  constexpr int BM = 32 * MTW, TN = 16 * NJ * WN;
  constexpr int AB = BM / 16;          // 1 KB blocks of A per stage (16 rows each)
  constexpr int WB = TN / 16;          // 1 KB blocks of W per stage (32 k-rows x TN columns)
  constexpr int NB = AB + WB;
  constexpr int LW = (NB + NWV - 1) / NWV;  // loads per wave per step
  constexpr int RB = TN * 2;           // bytes per W k-row
  constexpr int SB = NB * 1024;        // bytes per stage
  static_assert(S >= 2 && S <= 4, "2 to 4 LDS stages");
  __shared__ __attribute__((aligned(1024))) unsigned char st0[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[S > 2 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char st3[S > 3 ? SB : 16];
  auto stage = [&](int i) -> unsigned char* { return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : st3; };

  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WN, wn = w % WN;
  const int NT = Ncols / TN;
  int n_act = n_active[0];
  if (n_act > N) n_act = N;
  const int64_t tiles = (int64_t)n_act * mch * NT;
  const int nx = (gridDim.x % kDmaXcds == 0) ? kDmaXcds : 1;
  const int64_t per_x = (tiles + nx - 1) / nx;
  const int64_t local = blockIdx.x / nx;
  const int64_t tile = (int64_t)(blockIdx.x % nx) * per_x + local;
  if (local >= per_x || tile >= tiles) return;

  // tile -> (active expert a, m-chunk mc, column block nt); up to 8 m-chunks
  // of an expert walk the column blocks together (shared panels in L2)
  const int64_t per_e = (int64_t)mch * NT;
  const int a = (int)(tile / per_e);
  const int rr = (int)(tile - (int64_t)a * per_e);
  const int GM = mch < 8 ? mch : 8;
  const int grp = rr / (GM * NT);
  const int gm_here = (mch - grp * GM) < GM ? (mch - grp * GM) : GM;
  const int in_g = rr - grp * GM * NT;
  const int mc = grp * GM + in_g % gm_here;
  const int nt = in_g / gm_here;

  const int e = __builtin_amdgcn_readfirstlane(active[a]);
  if (e < 0 || e >= N) return;
  int kept = __builtin_amdgcn_readfirstlane(kept_count[e]);
  if (kept > C) kept = C;
  const int m0 = mc * BM;
  int rows = kept - m0;
  if (rows <= 0) return;
  if (rows > BM) rows = BM;
  const int n0 = nt * TN;
  const int ksteps = K >> 5;

  const __amdgpu_buffer_rsrc_t ares = gather != nullptr ? dma_rsrc(A, a_rows * K * 2)
                                                        : dma_rsrc(A + ((int64_t)e * C + m0) * K, (int64_t)rows * K * 2);
  const __amdgpu_buffer_rsrc_t wres = dma_rsrc(W + (int64_t)e * K * Ncols, (int64_t)K * Ncols * 2);

  // the LW blocks this wave loads every step (block w + NWV i; past NB it
  // repeats block w + NWV (i - 1): same bytes to the same place), as lane offsets
  int voff[LW], lds_blk[LW];
  bool is_a[LW];
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    int j = w + NWV * i;
    if (j >= NB) j -= NWV;
    lds_blk[i] = j * 1024;
    is_a[i] = j < AB;
    if (j < AB) {
      const int r = 16 * j + (lane >> 2), q = (lane & 3) ^ a_swz(r);
      const int64_t src = r < rows ? (gather != nullptr ? (int64_t)gather[(int64_t)e * C + m0 + r] : (int64_t)r) : 0;
      voff[i] = r < rows ? (int)((src * K + q * 8) * 2) : 0x7ffffff0;
    } else {
      const int o = (j - AB) * 1024 + lane * 16;
      const int k = o / RB, pc = (o % RB) >> 4, lc = pc ^ w_swz(k);
      voff[i] = (k * Ncols + n0 + lc * 8) * 2;
    }
  }
  // branch-free issue: the descriptor and the per-step offset of each load are
  // wave-uniform selects (a branch would split the loop into blocks and the
  // compiler's wait counts would then drain the loads in flight)
  const int a_step = 64, w_step = 32 * Ncols * 2;
  auto issue = [&](int st, int s) {
    const int sc = s < ksteps ? s : ksteps - 1;  // past the end: re-read the last step (cache hit)
    unsigned char* base = stage(st);
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      const __amdgpu_buffer_rsrc_t rs = is_a[i] ? ares : wres;
      const int so = sc * (is_a[i] ? a_step : w_step);
      if (WNT && !is_a[i])
        dma16_nt(rs, base + lds_blk[i], voff[i], so);
      else
        dma16(rs, base + lds_blk[i], voff[i], so);
    }
  };

  // fragment addresses inside a stage
  int a_rd[MTW], b_rd[NJ][2];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt) {
    const int r = wm * (BM / 2) + mt * 16 + c;
    a_rd[mt] = r * 64 + ((kg ^ a_swz(r)) << 4);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 8 * kg + 4 * h + (c >> 2);
      const int n = wn * 16 * NJ + 16 * j + 4 * (c & 3);
      b_rd[j][h] = AB * 1024 + k * RB + (((n >> 3) ^ w_swz(k)) << 4) + ((n >> 2) & 1) * 8;
    }

  f32x4 acc[MTW][NJ];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // 16-row m-tiles of this wave that hold a filled slot: an expert with fewer
  // rows than the tile skips the MFMAs (and A reads) of its empty m-tiles
  int live_mt = (rows - wm * (BM / 2) + 15) >> 4;
  live_mt = live_mt < 0 ? 0 : live_mt > MTW ? MTW : live_mt;
  live_mt = __builtin_amdgcn_readfirstlane(live_mt);
  auto compute = [&](int st) {
    const unsigned char* base = stage(st);
    u32x4 bf[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const u32x2 l2 = lds_read_tr16(base + b_rd[j][0]), h2 = lds_read_tr16(base + b_rd[j][1]);
      bf[j] = u32x4{l2[0], l2[1], h2[0], h2[1]};
    }
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      if (mt < live_mt) {
        const u32x4 af = *reinterpret_cast<const u32x4*>(base + a_rd[mt]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[mt][j] = mfma_bf16_16x16x32(af, bf[j], acc[mt][j]);
      }
    }
  };
  // this wave's loads of the oldest in-flight step have landed and its reads
  // of the previous stage are done; then the barrier (no fence: the other
  // steps' loads stay in flight)
  auto step_sync = [&]() {
    SWM_WAIT_VMCNT_LGKM0((S - 2) * LW);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

#pragma unroll
  for (int s0 = 0; s0 < S - 1; ++s0) issue(s0, s0);
  int it = 0;
  for (; it + S <= ksteps; it += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      step_sync();
      issue((u + S - 1) % S, it + u + S - 1);  // into the stage computed one step ago
      compute(u);
    }
  }
#pragma unroll
  for (int u = 0; u < S - 1; ++u) {  // the last ksteps % S steps
    if (it + u < ksteps) {
      step_sync();
      issue((u + S - 1) % S, it + u + S - 1);
      compute(u);
    }
  }

  // no load may still be writing this workgroup's LDS when it exits
  SWM_WAIT_VMCNT_LGKM0(0);
  __syncthreads();  // every wave is done with the stages: they now stage the output

  // A lane holds rows 4 kg + i of each 16-row tile and column c of each
  // 16-column tile, so direct stores would write 32 bytes per row and
  // instruction.  Each 16-row slice of the wave's tile goes through its own LDS
  // region instead (rows padded to 16 NJ * 2 + 16 bytes: the four kg row groups
  // land on different banks) and leaves as 16-byte non-temporal stores that
  // cover whole 128-byte lines (4 rows x 32 NJ bytes per instruction).
  constexpr int ROWB = 32 * NJ + 16;
  static_assert(NWV * 16 * ROWB <= SB, "the output staging fits one LDS stage");
  unsigned char* ost = st0 + w * 16 * ROWB;
  constexpr int CH = 2 * NJ;  // 16-byte chunks per staged row
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float v = acc[mt][j][i];
        if (relu) v = fmaxf(v, 0.f);
        *reinterpret_cast<uint16_t*>(ost + (kg * 4 + i) * ROWB + (16 * j + c) * 2) = (uint16_t)f2bf(v);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q0 = 0; q0 < 16 * CH; q0 += 64) {
      const int q = q0 + lane, r = q / CH, ch = q - r * CH;
      const int rl = wm * (BM / 2) + mt * 16 + r;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ost + r * ROWB + ch * 16);
      if constexpr (CMB) {
        if (rl < rows) combine_piece(cmb, v, (int64_t)m0 + rl, n0 + wn * 16 * NJ + ch * 8, Ncols);
      } else if (rl < rows) {
        __builtin_nontemporal_store(
            v, reinterpret_cast<u32x4*>(out + ((int64_t)e * C + m0 + rl) * Ncols + n0 + wn * 16 * NJ + ch * 8));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the next slice overwrites the region
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <int MTW, int NJ, int S, int WN = 2>
static hipError_t launch_dma(const void* A, const void* W, void* out, const int32_t* kept, const int32_t* active,
                             const int32_t* n_active, int N, int C, int K, int Ncols, int relu, hipStream_t st,
                             const int32_t* gather, int64_t a_rows, const CombineArgs* cmb = nullptr) {
  constexpr int BM = 32 * MTW, TN = 16 * NJ * WN;
  const int mch = (C + BM - 1) / BM;
  int64_t grid = (int64_t)N * mch * (Ncols / TN);
  grid = (grid + kDmaXcds - 1) / kDmaXcds * kDmaXcds;
  const auto* a = static_cast<const uint16_t*>(A);
  const auto* w = static_cast<const uint16_t*>(W);
  auto* o = static_cast<uint16_t*>(out);
  // one m-chunk per expert: each weight panel is streamed by exactly one tile
  if (cmb != nullptr && cmb->y != nullptr)
    hipLaunchKernelGGL((ffn_tile_dma<MTW, NJ, S, false, WN, true>), dim3((unsigned)grid), dim3(128 * WN), 0, st, a, w,
                       o, kept, active, n_active, N, C, K, Ncols, relu, mch, gather, a_rows, *cmb);
  else if (mch == 1)
    hipLaunchKernelGGL((ffn_tile_dma<MTW, NJ, S, true, WN, false>), dim3((unsigned)grid), dim3(128 * WN), 0, st, a,
                       w, o, kept, active, n_active, N, C, K, Ncols, relu, mch, gather, a_rows, CombineArgs{});
  else
    hipLaunchKernelGGL((ffn_tile_dma<MTW, NJ, S, false, WN, false>), dim3((unsigned)grid), dim3(128 * WN), 0, st, a,
                       w, o, kept, active, n_active, N, C, K, Ncols, relu, mch, gather, a_rows, CombineArgs{});
  return hipGetLastError();
}

// Tiles need K and Ncols to be multiples of 256 (whole 32-deep steps in
// groups of 8, whole 128- or 256-column blocks).
bool tiled_ffn_applies(int C, int d, int dff) { return C > 64 && d % 256 == 0 && dff % 256 == 0; }

// 128 < C <= 160: one m-chunk per expert (each weight panel is streamed
// once).  With Ncols a multiple of 512, 160 x 512 tiles on 8 waves (2 x 4,
// 80 x 128 each) and 3 stages: every token-row block staged in LDS feeds twice
// as many weight columns, so the CU moves fewer bytes per weight byte (the
// 128-expert large layer, back-to-back launches: GEMM 1 1.72 ms against 1.80,
// GEMM 2 1.91 ms against 2.15-2.20 for 160 x 256 on 4 waves, which in turn took
// GEMM 1 from 2.83 ms with 160 x 128).  Otherwise 160 x 256 on 4 waves with 2
// stages.  64 < C <= 96: 96 x 256 tiles with 2 stages (top-2 on the base
// layer, C = 80: 132 us per launch against 138 us with 128 x 256 x 3 and
// 135-145 us for the other shapes tried).  128 x 256 tiles with 3 stages
// otherwise.  The dense shared expert runs that tile on 8 waves (2 x 4, 64 x
// 64 each; two workgroups per CU, four waves per SIMD): the large layer's step
// went from 6.25 to 6.04 ms against 4 waves (A/B in one process; 6.13 with 2
// stages, 6.06 with 160 x 256 on 8 waves for GEMM 1).  Timed alone, back to back,
// 128 x 512 and 160 x 256 on 8 waves had been within +-5% of the 4-wave tile.
hipError_t launch_tiled_dma(const void* A, const void* W, void* out, const int32_t* kept, const int32_t* active,
                            const int32_t* n_active, int N, int C, int K, int Ncols, int relu, hipStream_t st,
                            const int32_t* gather, int64_t a_rows, const CombineArgs* cmb) {
  if (cmb != nullptr && cmb->y != nullptr) {  // the dense second GEMM with the combine
    if (N != 1) return hipErrorInvalidValue;
    return launch_dma<4, 4, 3, 4>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, st, gather, a_rows, cmb);
  }
  if (C > 128 && C <= 160) {
    if (Ncols % 512 == 0)
      return launch_dma<5, 8, 3, 4>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, st, gather, a_rows);
    return launch_dma<5, 8, 2>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, st, gather, a_rows);
  }
  if (C > 64 && C <= 96)
    return launch_dma<3, 8, 2>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, st, gather, a_rows);
  if (N == 1)  // the dense shared expert: 128 x 256 on 8 waves
    return launch_dma<4, 4, 3, 4>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, st, gather, a_rows);
  return launch_dma<4, 8, 3>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, st, gather, a_rows);
}

}  // namespace swm
