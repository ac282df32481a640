// Expert FFN: out[e, s] = ReLU(in[e, s] . W1[e]) . W2[e] over the filled slots
// of the active experts only.
//
// Source: "Top-1 Routing" page, Key parameters and compute (each expert is a
// two-layer FFN, biases ignored; 2 x d_model x d_ff weights per expert); the
// activation is ReLU.  "MoE expert capacity factor and token dropping" page,
// Where capacity comes from (the grouped GEMM runs on the fixed [N, C, d]
// buffers).
//
// bf16 kernel (both GEMMs): a weight-streaming grouped GEMM on MFMA
// v_mfma_f32_16x16x32_bf16.  With at most C tokens per expert the GEMMs read
// every weight byte once for a few dozen FLOPs, so they are bound by HBM on the
// weights; the kernel is built to stream them:
//  * W is row-major [K][Ncols] (Ncols contiguous), but an MFMA operand wants
//    8 consecutive k per lane.  Lane l (c = l & 15, kg = l >> 4) loads the 8
//    bytes at columns 4c..4c+3 of the 8 rows 8kg..8kg+7 of a 32 x 64 weight
//    block (full 128-byte row segments across the wave), then transposes that
//    8 x 4 bf16 tile in registers.  Column j of the tile becomes the B operand
//    of MFMA j, whose 16 output columns are the physical columns 4c + j: the
//    weights never touch LDS, and the 4 accumulators of a lane hold 4
//    consecutive output columns of one row, so results leave as 8-byte stores.
//  * A = token rows (k contiguous), 16 rows per MFMA tile, up to MT tiles per
//    item.  Rows at or beyond kept_count are neither loaded (they read as zero
//    through the buffer descriptor) nor stored, and items beyond kept_count are
//    skipped, so empty capacity slots cost nothing.  The hidden matrix that the
//    first GEMM writes for the second is fragment-blocked (see hblk_pos) unless
//    the caller keeps it.
//  * Work item = (active expert, 64-column block, m-chunk of MT*16 rows).  The
//    KW waves that share an item (1, 2 or 4, chosen on the device from n_active
//    so that every wave slot of the persistent grid is busy) take every KW-th
//    32-deep k-step and meet in LDS (fixed-order sum); with KW == 1 a wave owns
//    its item.  Each wave keeps STAGES weight blocks in flight in a register
//    ring and loads its A fragments one step ahead; the k-loop is branch-free
//    so that the compiler's wait counts keep the ring full.
// No reduction ever crosses workgroups, so no agent-scope fences (which write
// back and invalidate whole L2 caches on this multi-XCD part) are needed.
// fp32 kernel: plain fp32 FMA, one workgroup per (slot row, expert).
#include "active_list.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

constexpr int kOutOfRange = 0x7ffffff0;  // buffer lane offset that reads as zero
constexpr int kXcds = 8;                  // accelerator complex dies of an MI355X

// raw buffer resource over `bytes` bytes from p (dword 3 is the gfx9 raw-buffer format)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// cache policy of the weight stream: nt (non-temporal).  Every weight byte is
// read once per launch, so it should not evict what is reused (the token rows,
// the outputs).  Measured on the base layer: 125 -> 123 us per launch; decode
// batch 49 -> 46 us.  A layer whose active weights fit the 256 MB memory-side
// cache (17 experts, 160 MB) loses its reuse across back-to-back launches
// instead (20.5 -> 25.2 us per launch).
constexpr int kWeightCpol = 2;  // the nt bit of the buffer load's cache-policy operand

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// weight stream: read once, so it may carry a streaming cache policy
__device__ __forceinline__ u32x4 buffer_load16_w(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kWeightCpol));
}

__device__ __forceinline__ u32x2 buffer_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kWeightCpol));
}


__device__ __forceinline__ u32x2 pack4(const float (&v)[4], bool relu) {
  u32x2 o;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float lo = v[2 * q], hi = v[2 * q + 1];
    if (relu) {
      lo = fmaxf(lo, 0.f);
      hi = fmaxf(hi, 0.f);
    }
    o[q] = pack_bf2(lo, hi);
  }
  return o;
}

__device__ __forceinline__ u32x4 pack8(const float (&v)[8], bool relu) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float lo = v[2 * q], hi = v[2 * q + 1];
    if (relu) {
      lo = fmaxf(lo, 0.f);
      hi = fmaxf(hi, 0.f);
    }
    o[q] = pack_bf2(lo, hi);
  }
  return o;
}



// Waves of one workgroup that share a work item along K (1, 2 or 4), the same
// in every workgroup of a launch: the smallest KW that gives every wave slot
// of the grid at least one task, else the largest allowed (every wave keeps at
// least 4 k-steps).  A K split costs an LDS reduction and a barrier per item;
// measured on the 128-expert base layer, a partly filled second round of whole
// items beats more rounds of split items (GEMM 1: 119 us with KW = 1 against
// 135 us with KW = 2), while leaving a quarter of the slots idle does not (GEMM
// 2: 159 us with KW = 1 against 137 us with KW = 2).
__device__ __forceinline__ int waves_per_item(int64_t base, int64_t wave_slots, int waves, int ksteps) {
  int best = 1;
  for (int kw = 1; kw <= waves; kw *= 2) {
    if (kw > 1 && ksteps < kw * 4) break;
    best = kw;
    if (base * kw >= wave_slots) break;
  }
  return best;
}

// One launch computes out = act(A . W) over the filled slots of the active
// experts: phase 1 (K = d_model, Ncols = d_ff, ReLU) or phase 2 (K = d_ff,
// Ncols = d_model).  A work item is (active expert, 64-column block, m-chunk of
// MT*16 rows); the KW waves that share an item take every KW-th 32-deep k-step
// and meet in LDS; with KW == 1 a wave owns its item and stores directly.  Each
// wave keeps STAGES weight blocks in flight (register ring) and its A fragments
// one step ahead.
// J = columns per lane (4: 64-column waves with 8-byte loads; 8: 128-column
// waves with 16-byte loads)
template <int J>
struct WRow;
template <>
struct WRow<4> {
  typedef u32x2 type;
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, int v, int s) { return buffer_load8(r, v, s); }
  static __device__ __forceinline__ void transpose(const type (&in)[8], u32x4 (&out)[4]) { transpose8x4(in, out); }
};
template <>
struct WRow<8> {
  typedef u32x4 type;
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, int v, int s) { return buffer_load16_w(r, v, s); }
  static __device__ __forceinline__ void transpose(const type (&in)[8], u32x4 (&out)[8]) { transpose8x8(in, out); }
};

// Output rows leave with non-temporal stores: written once, read once by the
// next launch.  Measured per launch on the base layer: GEMM 1 114.9 -> 110.0 us,
// GEMM 2 128.1 -> 116.9 us (the write stream disturbs the weight stream less).
template <int J>
__device__ __forceinline__ void store_row(uint16_t* p, const float (&v)[J], bool relu);
template <>
__device__ __forceinline__ void store_row<4>(uint16_t* p, const float (&v)[4], bool relu) {
  __builtin_nontemporal_store(pack4(v, relu), reinterpret_cast<u32x2*>(p));
}
template <>
__device__ __forceinline__ void store_row<8>(uint16_t* p, const float (&v)[8], bool relu) {
  __builtin_nontemporal_store(pack8(v, relu), reinterpret_cast<u32x4*>(p));
}

// Fragment-blocked hidden matrix.  Between the two GEMMs the hidden rows of an
// expert are stored as 1 KB blocks, one per (32-deep k-step, 16-row tile):
// block (s, t) of expert e starts at element (e * tiles * 16 * d_ff) +
// (s * tiles + t) * 512 and holds the 16 rows x 32 k of that step and tile as
// 16-byte chunks (row r, k-chunk q = k / 8 mod 4) at chunk position
// hblk_pos(r, q).  The second GEMM's A load of a step is then one contiguous
// 1 KB read per tile (lane (c, kg) reads chunk hblk_pos(c, kg)) instead of 16
// row segments of 64 bytes 2 d_ff bytes apart, and the first GEMM's stores
// (lane (c, g) holds rows 4g + i and chunk c mod 4) still cover whole 256-byte
// runs per instruction: for a fixed i the 16 lanes of a block write positions
// 16i .. 16i + 15.
__device__ __forceinline__ int hblk_pos(int r, int q) { return (r & 3) * 16 + (r >> 2) * 4 + q; }

template <int MT, int WAVES, int STAGES, int J>
__device__ __forceinline__ void ffn_stream(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                           uint16_t* __restrict__ out, const int32_t* __restrict__ kept_count,
                                           const int32_t* __restrict__ active, int n_act, int N, int C, int K,
                                           int Ncols, int relu, int mch, float* red,
                                           const int32_t* __restrict__ gather, int64_t a_rows, int a_tiles,
                                           int o_tiles) {
  constexpr int COLS = 16 * J;  // output columns per item
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, kg = lane >> 4;
  // wave index as a wave-uniform (scalar) value: everything derived from it -- item,
  // expert, buffer descriptors, row offsets -- then lives in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NCB = Ncols / COLS;
  const int ksteps = K >> 5;
  const int64_t base = (int64_t)n_act * NCB * mch;
  if (base <= 0) return;
  const int KW = waves_per_item(base, (int64_t)gridDim.x * WAVES, WAVES, ksteps);
  const int groups = WAVES / KW;
  const int g = w / KW, kw = w - g * KW;
  // Workgroups are dealt to the 8 XCDs round-robin (blockIdx % 8).  Each XCD
  // takes one contiguous range of the expert-major item list, so the column
  // blocks of an expert -- which all read its activation rows -- share one L2.
  const int nx = (gridDim.x % kXcds == 0) ? kXcds : 1;
  const int xcd = blockIdx.x % nx;
  const int64_t slots_x = (int64_t)(gridDim.x / nx) * groups;
  const int64_t per_x = (base + nx - 1) / nx;
  const int64_t rounds = (per_x + slots_x - 1) / slots_x;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int nk = (ksteps - kw + KW - 1) / KW;  // my k-steps: kw, kw + KW, ...

  for (int64_t round = 0; round < rounds; ++round) {
    const int64_t local = round * slots_x + (int64_t)(blockIdx.x / nx) * groups + g;
    const int64_t item = xcd * per_x + local;
    int rows = 0, e = 0, cb = 0, m0 = 0;
    if (local < per_x && item < base) {
      const int mc = (int)(item % mch);
      const int64_t r = item / mch;
      cb = (int)(r % NCB);
      const int a = (int)(r / NCB);
      e = __builtin_amdgcn_readfirstlane(active[a]);
      if (e >= 0 && e < N) {
        m0 = mc * MT * 16;
        int kept = __builtin_amdgcn_readfirstlane(kept_count[e]);
        if (kept > C) kept = C;
        rows = kept - m0;
        if (rows > MT * 16) rows = MT * 16;
      }
    }
    const int mtc = rows > 0 ? (rows + 15) >> 4 : 0;  // uniform across the wave

    f32x4 acc[MT][J];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < J; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (mtc > 0) {
      // Buffer loads: one 32-bit lane offset per operand, the per-row and per-step
      // offsets are wave-uniform SGPR values.  A rows at or beyond `rows` get a lane
      // offset past the descriptor's extent, so they read as zeros.
      const __amdgpu_buffer_rsrc_t wres = make_rsrc(W + (int64_t)e * K * Ncols, (int64_t)K * Ncols * 2);
      // gather != NULL: A is the token matrix [a_rows, K] and row r of the
      // expert's buffer is token gather[e * C + r] (the dispatch folded in)
      // a_tiles > 0: A is the hidden matrix in the fragment-blocked layout, a_tiles
      // 16-row tiles per expert
      const int64_t a_rows_e = (int64_t)a_tiles * 16;
      const __amdgpu_buffer_rsrc_t ares =
          a_tiles > 0 ? make_rsrc(A + (int64_t)e * a_rows_e * K, a_rows_e * K * 2)
          : gather != nullptr ? make_rsrc(A, a_rows * K * 2)
                              : make_rsrc(A + ((int64_t)e * C + m0) * K, (int64_t)rows * K * 2);
      const int w_voff = ((kw * 32 + kg * 8) * Ncols + cb * COLS + c * J) * 2;
      const int w_row = Ncols * 2;
      const int w_step = KW * 32 * Ncols * 2;
      int a_voff[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int rr = mt * 16 + c;
        if (a_tiles > 0) {  // block (k-step kw, tile m0/16 + mt): row c, k-chunk kg at hblk_pos(c, kg)
          a_voff[mt] = rr < rows ? (kw * a_tiles + (m0 >> 4) + mt) * 1024 + hblk_pos(c, kg) * 16 : kOutOfRange;
        } else {
          const int64_t src = gather != nullptr && rr < rows ? gather[(int64_t)e * C + m0 + rr] : rr;
          a_voff[mt] = rr < rows ? (int)((src * K + kw * 32 + kg * 8) * 2) : kOutOfRange;
        }
      }
      const int a_step = a_tiles > 0 ? KW * a_tiles * 1024 : KW * 32 * 2;

      // The k-loop has no data-dependent branches (the waitcnt pass would drain
      // every load at each join).  The step count is padded to a multiple of
      // STAGES; prefetches past the last step re-read the last weight block (an L2
      // hit) and padding steps multiply a zero A fragment.  The zero is selected
      // where the fragment is used: a select right after the load would make the
      // load wait for itself, and with it for every load issued before it.
      auto load_a = [&](u32x4 (&dst)[MT], int step) {
        const int so = (step < nk ? step : nk - 1) * a_step;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) dst[mt] = buffer_load16(ares, a_voff[mt], so);
      };
      typedef typename WRow<J>::type wrow_t;
      auto load_w = [&](wrow_t (&dst)[8], int step) {
        const int so = (step < nk ? step : nk - 1) * w_step;
#pragma unroll
        for (int r = 0; r < 8; ++r) dst[r] = WRow<J>::load(wres, w_voff, so + r * w_row);
      };
      // A fragments and weight blocks share one ring: step s's loads are issued
      // together STAGES - 1 steps ahead.  Loads retire in order, so an A load
      // issued later than the weights (say one step ahead) would make the wait
      // for it drain the weight ring as well.
      u32x4 abuf[STAGES][MT];
      wrow_t buf[STAGES][8];
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s) {
        load_w(buf[s], s);
        load_a(abuf[s], s);
      }

      const int nk_pad = (nk + STAGES - 1) / STAGES * STAGES;
      for (int it = 0; it < nk_pad; it += STAGES) {
#pragma unroll
        for (int u = 0; u < STAGES; ++u) {
          const int cur = it + u;
          load_w(buf[(u + STAGES - 1) % STAGES], cur + STAGES - 1);
          load_a(abuf[(u + STAGES - 1) % STAGES], cur + STAGES - 1);
          // keep the prefetches ahead of this step's math: the scheduler would sink
          // them below the MFMAs, and the next step would then wait for them
          __builtin_amdgcn_sched_barrier(0);
          const bool live = cur < nk;
          u32x4 af[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) af[mt] = live ? abuf[u][mt] : zero;
          u32x4 bt[J];
          WRow<J>::transpose(buf[u], bt);
#pragma unroll
          for (int j = 0; j < J; ++j)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt][j] = mfma_bf16_16x16x32(af[mt], bt[j], acc[mt][j]);
        }
      }
    }

    // where this lane's J columns of item row rl go: row-major [N, C, Ncols], or
    // (o_tiles > 0) the fragment-blocked layout that the next GEMM reads
    auto out_at = [&](int rl) -> uint16_t* {
      const int col0 = cb * COLS + c * J;
      const int r = m0 + rl;
      if (o_tiles > 0)
        return out + (int64_t)e * o_tiles * 16 * Ncols + ((int64_t)(col0 >> 5) * o_tiles + (r >> 4)) * 512 +
               hblk_pos(r & 15, (col0 & 31) >> 3) * 8 + (col0 & 7);
      return out + ((int64_t)e * C + r) * Ncols + col0;
    };
    if (KW == 1) {
      // this wave owns the item: lane holds rows 4*kg + i, columns J*c .. J*c + J-1
      if (mtc > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rl = mt * 16 + kg * 4 + i;
            if (mt < mtc && rl < rows) {
              float v[J];
#pragma unroll
              for (int j = 0; j < J; ++j) v[j] = acc[mt][j][i];
              store_row<J>(out_at(rl), v, relu);
            }
          }
        }
      }
    } else {
      // the KW waves of a group sum their partials in LDS (fixed order); wave kw
      // of the group finishes rows 4*kg + i for i = kw, kw + KW, ...
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[((w * 4 + i) * J + j) * 64 + lane] = acc[mt][j][i];
        __syncthreads();
        if (mt < mtc) {
          for (int i = kw; i < 4; i += KW) {
            float v[J];
#pragma unroll
            for (int j = 0; j < J; ++j) {
              float sum = 0.f;
              for (int q = 0; q < KW; ++q) sum += red[(((g * KW + q) * 4 + i) * J + j) * 64 + lane];
              v[j] = sum;
            }
            const int rl = mt * 16 + kg * 4 + i;
            if (rl < rows) store_row<J>(out_at(rl), v, relu);
          }
        }
        __syncthreads();
      }
    }
  }
}

// 128-column work items (16-byte weight loads, J = 8) unless, even at the
// largest K split, they would give fewer than 2/5 of the grid's wave slots a
// task; then 64-column items (twice as many).  The threshold sits between
// measured launches: 128-column items won on GEMM 2 of the base layer (150
// tasks per 100 slots: 127 us against 140 us) and on both GEMMs of the
// 384-expert decode layer with 14 experts active (44 and 88 per 100 slots: 47
// against 48-50 us), and lost on GEMM 2 of the skewed layer with 17 experts
// active (20 per 100 slots: 22.4 against 18.9 us).  The choice needs n_active,
// so it is taken on the device; JMAX = 4 compiles the 64-column path only.
template <int MT, int WAVES, int STAGES, int JMAX>
__global__ __launch_bounds__(WAVES * 64, 2) void ffn_gemm_bf16(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, uint16_t* __restrict__ out,
    const int32_t* __restrict__ kept_count, const int32_t* __restrict__ active, const int32_t* __restrict__ n_active,
    int N, int C, int K, int Ncols, int relu, int mch, const int32_t* __restrict__ gather, int64_t a_rows, int a_tiles,
    int o_tiles, ActiveFromKept afk) {
  __shared__ float red[WAVES * 4 * JMAX * 64];
  __shared__ int s_act[1024];
  __shared__ int wsum[16];
  __shared__ double sl[16];
  int n_act;
  if (afk.kept != nullptr) {
    n_act = active_from_kept<WAVES * 64>(afk, N, s_act, wsum, sl);
    active = s_act;
  } else {
    n_act = n_active[0];
  }
  if (n_act > N) n_act = N;
  if (JMAX == 8 && Ncols % 128 == 0 &&
      (int64_t)n_act * (Ncols / 128) * mch * WAVES * 5 >= (int64_t)gridDim.x * WAVES * 2)
    ffn_stream<MT, WAVES, STAGES, JMAX>(A, W, out, kept_count, active, n_act, N, C, K, Ncols, relu, mch, red, gather,
                                        a_rows, a_tiles, o_tiles);
  else
    ffn_stream<MT, WAVES, STAGES, 4>(A, W, out, kept_count, active, n_act, N, C, K, Ncols, relu, mch, red, gather,
                                     a_rows, a_tiles, o_tiles);
}

__global__ __launch_bounds__(256) void ffn_gemm_f32(const float* __restrict__ A, const float* __restrict__ W,
                                                    float* __restrict__ out, const int32_t* __restrict__ kept_count,
                                                    const int32_t* __restrict__ active,
                                                    const int32_t* __restrict__ n_active, int N, int C, int K,
                                                    int Ncols, int relu, const int32_t* __restrict__ gather) {
  const int a = blockIdx.y;
  if (a >= n_active[0]) return;
  const int e = active[a];
  if (e < 0 || e >= N) return;
  const int row = blockIdx.x;
  if (row >= kept_count[e] || row >= C) return;
  const int64_t src = gather != nullptr ? (int64_t)gather[(int64_t)e * C + row] : (int64_t)e * C + row;
  const float* ar = A + src * K;
  const float* wb = W + (int64_t)e * K * Ncols;
  float* orow = out + ((int64_t)e * C + row) * Ncols;
  for (int col = threadIdx.x; col < Ncols; col += 256) {
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc = fmaf(ar[k], wb[(int64_t)k * Ncols + col], acc);
    orow[col] = relu ? fmaxf(acc, 0.f) : acc;
  }
}

__global__ void dense_plan(int32_t* kept, int32_t* active, int32_t* n_active, int32_t M) {
  if (threadIdx.x == 0) {
    kept[0] = M;
    active[0] = 0;
    n_active[0] = 1;
  }
}

// ----------------------------------------------------------------------------
// streaming GEMM launch shape: 4 waves per workgroup, a 2-deep register ring
constexpr int kStreamWaves = 4;
constexpr int kStreamStages = 2;

FfnPlan ffn_plan(int N, int C, int d, int dff, int dtype) {
  FfnPlan pl{};
  size_t off = 0;
  const size_t esz = dtype == 1 ? 2 : 4;
  int64_t h_rows = C;  // rows of the hidden matrix per expert
  if (dtype == 1) {
    pl.mt = C <= 16 ? 1 : C <= 32 ? 2 : C <= 48 ? 3 : 4;
    pl.mch = (C + pl.mt * 16 - 1) / (pl.mt * 16);
    pl.grid = 0;  // persistent grid: resident workgroups per CU x CUs, resolved at launch
    // fragment-blocked hidden matrix for the streaming GEMMs: every 16-row tile
    // of every expert is whole, and an expert's block stays under 2^31 bytes
    const int64_t tiles = (int64_t)pl.mch * pl.mt;
    if (!tiled_ffn_applies(C, d, dff) && tiles * 16 * dff * 2 < ((int64_t)1 << 31)) {
      pl.h_tiles = (int)tiles;
      h_rows = tiles * 16;
    }
  }
  pl.off_h = off;
  off = align_up(off + (size_t)N * h_rows * dff * esz);
  pl.bytes = off;
  return pl;
}

hipError_t launch_dense_plan(int32_t* kept, int32_t* active, int32_t* n_active, int32_t M, hipStream_t st) {
  hipLaunchKernelGGL(dense_plan, dim3(1), dim3(64), 0, st, kept, active, n_active, M);
  return hipGetLastError();
}

// resident workgroups of `kernel` on the whole device (occupancy x CUs), cached
// per (kernel, device)
static int persistent_grid(const void* kernel, int threads) {
  struct Entry {
    const void* kernel;
    int device, grid;
  };
  static thread_local Entry cache[16];
  static thread_local int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  for (int i = 0; i < used; ++i)
    if (cache[i].kernel == kernel && cache[i].device == dev) return cache[i].grid;
  int per_cu = 1, cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1) per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  const int grid = per_cu * cus;
  if (used < 16) cache[used++] = Entry{kernel, dev, grid};
  return grid;
}

template <int MT, int J>
static hipError_t launch_gemm(const void* A, const void* W, void* out, const int32_t* kept, const int32_t* active,
                              const int32_t* n_active, int N, int C, int K, int Ncols, int relu, int mch,
                              hipStream_t st, const int32_t* gather, int64_t a_rows, int a_tiles, int o_tiles,
                              const ActiveFromKept& afk) {
  constexpr int kWaves = kStreamWaves;
  auto kern = ffn_gemm_bf16<MT, kWaves, kStreamStages, J>;
  const int grid = persistent_grid(reinterpret_cast<const void*>(kern), kWaves * 64);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kWaves * 64), 0, st, static_cast<const uint16_t*>(A),
                     static_cast<const uint16_t*>(W), static_cast<uint16_t*>(out), kept, active, n_active, N, C, K,
                     Ncols, relu, mch, gather, a_rows, a_tiles, o_tiles, afk);
  return hipGetLastError();
}

// 128-column items are possible up to 3 row tiles (4 x 8 accumulator tiles
// would spill); the kernel picks 128- or 64-column items per launch
template <int MT>
static hipError_t launch_gemm_cols(const void* A, const void* W, void* out, const int32_t* kept,
                                   const int32_t* active, const int32_t* n_active, int N, int C, int K, int Ncols,
                                   int relu, int mch, hipStream_t st, const int32_t* gather, int64_t a_rows,
                                   int a_tiles, int o_tiles, const ActiveFromKept& afk) {
  if constexpr (MT <= 3) {
    if (Ncols % 128 == 0)
      return launch_gemm<MT, 8>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, mch, st, gather, a_rows,
                                a_tiles, o_tiles, afk);
  }
  return launch_gemm<MT, 4>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, mch, st, gather, a_rows, a_tiles,
                            o_tiles, afk);
}

static hipError_t gemm_bf16(const FfnPlan& pl, const void* A, const void* W, void* out, const int32_t* kept,
                            const int32_t* active, const int32_t* n_active, int N, int C, int K, int Ncols, int relu,
                            hipStream_t st, const int32_t* gather, int64_t a_rows, int a_tiles, int o_tiles,
                            const ActiveFromKept& afk = ActiveFromKept{}) {
  switch (pl.mt) {
    case 1: return launch_gemm_cols<1>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, pl.mch, st, gather,
                                       a_rows, a_tiles, o_tiles, afk);
    case 2: return launch_gemm_cols<2>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, pl.mch, st, gather,
                                       a_rows, a_tiles, o_tiles, afk);
    case 3: return launch_gemm_cols<3>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, pl.mch, st, gather,
                                       a_rows, a_tiles, o_tiles, afk);
    default: return launch_gemm_cols<4>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, pl.mch, st, gather,
                                        a_rows, a_tiles, o_tiles, afk);
  }
}

hipError_t launch_ffn(const FfnPlan& pl, const void* xin, const void* w1, const void* w2, int dtype, int N, int C, int d,
                      int dff, const int32_t* kept_count, const int32_t* active, const int32_t* n_active, void* xout,
                      char* ws, hipStream_t st, const int32_t* gather, int64_t a_rows, void* h_out,
                      const MxWeights* mx, const ActiveFromKept* afk, const CombineArgs* cmb) {
  void* h = h_out != nullptr ? h_out : static_cast<void*>(ws + pl.off_h);
  if (afk != nullptr && !ffn_stream_applies(dtype, C, d, dff, mx != nullptr)) return hipErrorInvalidValue;
  // the fused combine exists on the tiled path only (the caller checks tiled_ffn_applies)
  if (cmb != nullptr && cmb->y != nullptr && (dtype != 1 || mx != nullptr || !tiled_ffn_applies(C, d, dff)))
    return hipErrorInvalidValue;
  if (mx != nullptr)  // MXFP4 weights (bf16 activations; the caller checked mx_ffn_applies)
    return launch_ffn_mx(xin, *mx, N, C, d, dff, kept_count, active, n_active, xout, h, st, gather, a_rows,
                         afk != nullptr ? *afk : ActiveFromKept{});
  if (dtype == 0) {
    hipLaunchKernelGGL(ffn_gemm_f32, dim3((unsigned)C, (unsigned)N), dim3(256), 0, st, static_cast<const float*>(xin),
                       static_cast<const float*>(w1), static_cast<float*>(h), kept_count, active, n_active, N, C, d,
                       dff, 1, gather);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ffn_gemm_f32, dim3((unsigned)C, (unsigned)N), dim3(256), 0, st, static_cast<const float*>(h),
                       static_cast<const float*>(w2), static_cast<float*>(xout), kept_count, active, n_active, N, C,
                       dff, d, 0, nullptr);
    return hipGetLastError();
  }
  if (tiled_ffn_applies(C, d, dff)) {
    hipError_t e = launch_tiled_dma(xin, w1, h, kept_count, active, n_active, N, C, d, dff, 1, st, gather, a_rows);
    if (e != hipSuccess) return e;
    return launch_tiled_dma(h, w2, xout, kept_count, active, n_active, N, C, dff, d, 0, st, nullptr, 0, cmb);
  }
  // The hidden matrix stays in the library's workspace unless the caller keeps
  // it (training); then it is row-major [N, C, d_ff] as documented.  In the
  // workspace it takes the fragment-blocked layout (ffn_plan sizes it).
  const int tiles = h_out == nullptr ? pl.h_tiles : 0;
  hipError_t e = gemm_bf16(pl, xin, w1, h, kept_count, active, n_active, N, C, d, dff, 1, st, gather, a_rows, 0, tiles,
                           afk != nullptr ? *afk : ActiveFromKept{});
  if (e != hipSuccess) return e;
  return gemm_bf16(pl, h, w2, xout, kept_count, active, n_active, N, C, dff, d, 0, st, nullptr, 0, tiles, 0);
}

bool ffn_stream_applies(int dtype, int C, int d, int dff, bool mx) {
  return dtype == 1 && (mx ? mx_ffn_applies(C, d, dff) : !tiled_ffn_applies(C, d, dff));
}

}  // namespace swm
