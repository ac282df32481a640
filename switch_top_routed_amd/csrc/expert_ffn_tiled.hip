// Expert FFN for large per-expert row counts: an LDS-tiled MFMA GEMM.
//
// Same operation as the weight-streaming kernel (out = act(A . W) over the
// filled slots of the active experts; "Top-1 Routing" page, Key parameters and
// compute), used when an expert holds more than 64 rows (capacity C > 64) and
// for the always-on shared dense expert (N = 1, C = T rows).  There the work per
// weight byte is high enough that MFMA throughput and panel reuse matter:
//  * a workgroup (4 waves, 2 x 2) owns a BM x 256 output tile, BM = 32 * MTW
//    (128 or 192 rows), and walks K in 32-deep steps;
//  * per step the A rows (k contiguous) go to LDS as they are; the W block
//    (32 k-rows x 256 columns, columns contiguous) is loaded 8 bytes per lane
//    per row, transposed 8 x 4 in registers and written to LDS k-contiguous, so
//    every MFMA fragment is one ds_read_b128.  Both LDS tiles store 16-byte
//    chunks XOR-swizzled by row; the swizzle keeps the fragment reads, the A
//    stores and the transposed W stores free of bank conflicts whether the LDS
//    serves 8 lanes x 16 bytes or 16 lanes x 16 bytes per clock;
//  * the W columns are permuted in LDS so that MFMA j of a wave reads 16
//    consecutive LDS rows yet produces the physical columns 8c + j: a lane's 8
//    accumulators then hold 8 consecutive output columns (16-byte stores);
//  * global loads run P steps ahead of the MFMAs (register ring) and LDS is
//    double-buffered, one barrier per step;
//  * 128-row tiles fit in half the register file, so two workgroups share a
//    CU (two waves per SIMD): one wave's MFMAs then overlap the other's loads,
//    LDS traffic and barrier.  That beats a single 256-row workgroup per CU,
//    whose lone wave per SIMD runs its memory work and its MFMAs in series;
//  * tiles are dealt to the 8 XCDs in contiguous ranges and, inside an expert,
//    grouped 8 m-chunks at a time per column block, so that the workgroups
//    running together on one XCD share A and W panels in its L2.
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

namespace {

constexpr int kTileN = 256;
constexpr int kTiledXcds = 8;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 tload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ u32x2 tload8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// byte offset of 16-byte chunk q (0..3) of LDS row r (64 bytes per row).  The
// chunk is XORed with two parity bits of the row: bit 0 = r1 ^ r2, bit 1 =
// r1 ^ r3 ^ r6 (r_i = bit i of r), chosen by exhaustive search over linear
// swizzles so that 8 (and 16) consecutive lanes of every b128 access in this
// kernel cover distinct banks.
__device__ __forceinline__ int lds_swz(int r) {
  return (((r >> 1) ^ (r >> 2)) & 1) | ((((r >> 1) ^ (r >> 3) ^ (r >> 6)) & 1) << 1);
}
__device__ __forceinline__ int lds_off(int r, int q) { return r * 64 + ((q ^ lds_swz(r)) << 4); }

// LDS row of tile column col (0..32 NJ - 1) for waves of 16 NJ columns: wave
// half wn = col / (16 NJ), lane c = (col % (16 NJ)) / NJ, MFMA j = col % NJ
//   ->  row wn * 16 NJ + 16 j + c
template <int NJ>
__device__ __forceinline__ int col_row(int col) {
  const int cc = col % (16 * NJ);
  return (col - cc) + ((cc % NJ) << 4) + cc / NJ;
}

// row i of a lane's NJ accumulators as NJ bf16 (NJ / 2 dwords)
template <int NJ>
__device__ __forceinline__ void pack_row(const f32x4 (&acc)[NJ], int i, bool relu, uint32_t (&o)[NJ / 2]) {
#pragma unroll
  for (int q = 0; q < NJ / 2; ++q) {
    float lo = acc[2 * q][i], hi = acc[2 * q + 1][i];
    if (relu) {
      lo = fmaxf(lo, 0.f);
      hi = fmaxf(hi, 0.f);
    }
    o[q] = pack_bf2(lo, hi);
  }
}

// in[r] = 4 bf16 of k-row r (two per dword); out[j] = the 4 k-rows of column j
__device__ __forceinline__ void transpose4x4(const u32x2 (&in)[4], u32x2 (&out)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int dw = j >> 1, sh = (j & 1) * 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t a = (in[2 * h][dw] >> sh) & 0xffffu, b = (in[2 * h + 1][dw] >> sh) & 0xffffu;
      out[j][h] = a | (b << 16);
    }
  }
}

}  // namespace

// MTW m-tiles x NJ n-tiles of 16 x 16 per wave; the tile is BM = 32 MTW rows
// by TN = 32 NJ columns (NJ = 8: 256 columns, NJ = 4: 128 columns).  Tiles
// whose accumulators fit in a quarter of the register file run two
// workgroups per CU.
template <int MTW, int NJ, int P>
__global__ __launch_bounds__(256, (MTW * NJ <= 32 ? 2 : 1)) void ffn_tile_bf16(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, uint16_t* __restrict__ out,
    const int32_t* __restrict__ kept_count, const int32_t* __restrict__ active, const int32_t* __restrict__ n_active,
    int N, int C, int K, int Ncols, int relu, int mch, const int32_t* __restrict__ gather, int64_t a_rows) {
  static_assert(NJ == 4 || NJ == 8, "tile width 128 or 256 columns");
  static_assert(8 % P == 0, "prefetch depth divides the k-steps of a 256-multiple K");
  constexpr int BM = 32 * MTW;                 // tile rows (2 waves x MTW x 16)
  constexpr int TN = 32 * NJ;                  // tile columns (2 waves x 16 lanes x NJ)
  constexpr int ACH = (BM * 4 + 255) / 256;    // 16-byte A chunks per thread per step
  constexpr int BUF = (BM + TN) * 64;          // bytes per LDS buffer
  constexpr int WLD = NJ == 8 ? 8 : 4;         // W loads (8 bytes) per thread per step
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int NT = Ncols / TN;
  int n_act = n_active[0];
  if (n_act > N) n_act = N;
  const int64_t tiles = (int64_t)n_act * mch * NT;
  const int nx = (gridDim.x % kTiledXcds == 0) ? kTiledXcds : 1;
  const int64_t per_x = (tiles + nx - 1) / nx;
  const int64_t local = blockIdx.x / nx;
  const int64_t tile = (int64_t)(blockIdx.x % nx) * per_x + local;
  if (local >= per_x || tile >= tiles) return;

  // tile -> (active expert a, m-chunk mc, column block nt); inside an expert,
  // groups of up to 8 m-chunks walk the column blocks together
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

  // gather != NULL: A is the token matrix [a_rows, K], tile row r is token gather[e * C + m0 + r]
  const __amdgpu_buffer_rsrc_t ares = gather != nullptr ? tile_rsrc(A, a_rows * K * 2)
                                                        : tile_rsrc(A + ((int64_t)e * C + m0) * K, (int64_t)rows * K * 2);
  const __amdgpu_buffer_rsrc_t wres = tile_rsrc(W + (int64_t)e * K * Ncols, (int64_t)K * Ncols * 2);

  // A: chunk ch = tid + 256 i is 16-byte chunk ch % 4 of tile row ch / 4
  int a_voff[ACH], a_lds[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int ch = tid + i * 256, r = ch >> 2, q = ch & 3;
    const int64_t src = gather != nullptr && r < rows ? gather[(int64_t)e * C + m0 + r] : r;
    a_voff[i] = r < rows ? (int)((src * K + q * 8) * 2) : 0x7ffffff0;  // rows past `rows` read zero
    a_lds[i] = lds_off(r, q);
  }
  // W, 256 columns: thread (w, c, kg) loads k-rows 8 kg .. 8 kg + 7 of columns
  //   64 w + 4 c .. + 3, transposes 8 x 4 and writes four 16-byte k-chunks;
  // W, 128 columns: thread (kq = 2 w + (lane & 1), c4 = lane / 2) loads k-rows
  //   4 kq .. 4 kq + 3 of columns 4 c4 .. + 3, transposes 4 x 4 and writes four
  //   8-byte half-chunks (adjacent lanes fill the two halves of one chunk)
  int w_voff, b_lds[4];
  if (NJ == 8) {
    w_voff = ((kg * 8) * Ncols + n0 + w * 64 + c * 4) * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) b_lds[j] = BM * 64 + lds_off(col_row<NJ>(w * 64 + c * 4 + j), kg);
  } else {
    const int kq = 2 * w + (lane & 1), c4 = lane >> 1;
    w_voff = ((kq * 4) * Ncols + n0 + c4 * 4) * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) b_lds[j] = BM * 64 + lds_off(col_row<NJ>(c4 * 4 + j), kq >> 1) + (kq & 1) * 8;
  }

  u32x4 ra[P][ACH];
  u32x2 rw[P][WLD];
  auto load_step = [&](int slot, int s) {
    const int sc = s < ksteps ? s : ksteps - 1;  // past the end: re-read the last step (cache hit)
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra[slot][i] = tload16(ares, a_voff[i], sc * 64);
#pragma unroll
    for (int r = 0; r < WLD; ++r) rw[slot][r] = tload8(wres, w_voff, (sc * 32 + r) * Ncols * 2);
  };
  auto store_step = [&](int slot, int buf) {
    unsigned char* base = lds + buf * BUF;
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      if (i < ACH - 1 || BM * 4 % 256 == 0 || w < (BM * 4 % 256) / 64)  // wave-uniform tail
        *reinterpret_cast<u32x4*>(base + a_lds[i]) = ra[slot][i];
    if (NJ == 8) {
      u32x2 in8[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) in8[r] = rw[slot][r % WLD];
      u32x4 bt[4];
      transpose8x4(in8, bt);
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(base + b_lds[j]) = bt[j];
    } else {
      u32x2 in4[4], bt[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) in4[r] = rw[slot][r];
      transpose4x4(in4, bt);
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(base + b_lds[j]) = bt[j];
    }
  };

  f32x4 acc[MTW][NJ];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  int a_rd[MTW], b_rd[NJ];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt) a_rd[mt] = lds_off(wm * (BM / 2) + mt * 16 + c, kg);
#pragma unroll
  for (int j = 0; j < NJ; ++j) b_rd[j] = BM * 64 + lds_off(wn * 16 * NJ + 16 * j + c, kg);

  // register ring: slot s % P holds step s from its load (issued P steps
  // earlier) until it is written to LDS buffer s % 2 one step before its MFMAs.
  // K is a multiple of 256, so ksteps is a multiple of 8 and of P.
#pragma unroll
  for (int s0 = 0; s0 < P; ++s0) load_step(s0, s0);
  store_step(0, 0);
  __syncthreads();
  for (int it = 0; it < ksteps; it += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int s = it + u;
      // slot u held step s (in LDS since the last step): reload it with step s + P
      load_step(u, s + P);
      __builtin_amdgcn_sched_barrier(0);
      const unsigned char* base = lds + (u & 1) * BUF;
      u32x4 bf[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[j] = *reinterpret_cast<const u32x4*>(base + b_rd[j]);
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt) {
        const u32x4 af = *reinterpret_cast<const u32x4*>(base + a_rd[mt]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[mt][j] = mfma_bf16_16x16x32(af, bf[j], acc[mt][j]);
      }
      store_step((u + 1) % P, (u + 1) & 1);  // step s + 1 into the other buffer
      __syncthreads();
    }
  }

  // lane holds rows 4 kg + i of each 16-row tile, columns NJ c .. NJ c + NJ - 1 of its half
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = wm * (BM / 2) + mt * 16 + kg * 4 + i;
      uint32_t o[NJ / 2];
      pack_row<NJ>(acc[mt], i, relu != 0, o);
      uint16_t* dst = out + ((int64_t)e * C + m0 + rl) * Ncols + n0 + wn * 16 * NJ + c * NJ;
      if (rl < rows) {
        if (NJ == 8)
          *reinterpret_cast<u32x4*>(dst) = u32x4{o[0], o[1], o[2 % (NJ / 2)], o[3 % (NJ / 2)]};
        else
          *reinterpret_cast<u32x2*>(dst) = u32x2{o[0], o[1]};
      }
    }
  }
}

#ifndef SWM_TILE_P
#define SWM_TILE_P 4
#endif

template <int MTW, int NJ, int P>
static hipError_t launch_tiled(const void* A, const void* W, void* out, const int32_t* kept, const int32_t* active,
                               const int32_t* n_active, int N, int C, int K, int Ncols, int relu, hipStream_t st,
                               const int32_t* gather, int64_t a_rows) {
  constexpr int BM = 32 * MTW, TN = 32 * NJ;
  const int mch = (C + BM - 1) / BM;
  int64_t grid = (int64_t)N * mch * (Ncols / TN);
  grid = (grid + kTiledXcds - 1) / kTiledXcds * kTiledXcds;
  hipLaunchKernelGGL((ffn_tile_bf16<MTW, NJ, P>), dim3((unsigned)grid), dim3(256), 0, st,
                     static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W), static_cast<uint16_t*>(out), kept,
                     active, n_active, N, C, K, Ncols, relu, mch, gather, a_rows);
  return hipGetLastError();
}

bool tiled_ffn_applies(int C, int d, int dff) { return C > 64 && d % kTileN == 0 && dff % kTileN == 0; }

hipError_t launch_tiled_gemm(const void* A, const void* W, void* out, const int32_t* kept, const int32_t* active,
                             const int32_t* n_active, int N, int C, int K, int Ncols, int relu, hipStream_t st,
                             const int32_t* gather, int64_t a_rows) {
  // One m-chunk per expert where C allows (each weight panel is then streamed
  // once): 160 x 128 tiles (two workgroups per CU) for 128 < C <= 160, 192 x 256
  // tiles for 160 < C <= 192; 128 x 256 tiles, two workgroups per CU, otherwise.
  if (C > 128 && C <= 160)
    return launch_tiled<5, 4, SWM_TILE_P>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, st, gather, a_rows);
  if (C > 160 && C <= 192)
    return launch_tiled<6, 8, SWM_TILE_P>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, st, gather, a_rows);
  return launch_tiled<4, 8, 2>(A, W, out, kept, active, n_active, N, C, K, Ncols, relu, st, gather, a_rows);
}

}  // namespace swm
