// Expert FFN with MXFP4 weights (bf16 activations, fp32 accumulation), and the
// quantizer that produces them.
//
// The open-MoE routing comparison page (TL;DR, gpt-oss passage) reports MoE
// weights shipped in MXFP4 so that a large model fits one GPU; the format is
// the OCP Microscaling (MX) v1.0 one: blocks of 32 elements along the GEMM's
// reduction dimension share an E8M0 scale 2^E, elements are FP4 E2M1.  Layout:
// a weight W [E][K][Ncols] becomes codes [E][Ncols][K/2] (two elements per byte,
// lower index in the low nibble) and scales [E][Ncols][K/32] (bytes E + 127),
// so the reduction dimension is contiguous.
//
// For the weight-bound expert GEMM (few tokens per expert) a quarter of the
// bf16 weight bytes (plus 1/32 for the scales) streams from HBM.  Each lane
// loads, per output column and 128-deep step, one whole 32-element block (16
// code bytes) and its scale, and turns each 8-element group into an MFMA B
// fragment with the gfx950 conversion v_cvt_scalef32_pk_bf16_fp4 (byte `sel`
// of a dword: low nibble -> low bf16, high nibble -> high bf16, times the
// power-of-two scale; exact, as every product of an E2M1 value and 2^E is a
// bf16 value).  The reduction index is permuted identically in A and B: in
// sub-step q the lane group kg covers k = 32 kg + 8 q + 0..7, so a lane's B
// fragments all come from its own block and its A fragments from 64
// contiguous bytes of the token row.  Work items, the K split across waves and
// the output layout (4 consecutive columns per lane) follow the bf16
// weight-streaming kernel.
#include "active_list.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

namespace {

constexpr int kMxXcds = 8;
constexpr int kMxOOR = 0x7ffffff0;  // lane offset past any descriptor: reads zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 mx_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// default cache policy for the codes and scales as well: non-temporal loads
// were measured slower here (base layer 93 -> 108 us per launch)
__device__ __forceinline__ uint32_t mx_load4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

typedef __bf16 bf16x2_mx __attribute__((ext_vector_type(2)));
// 8 fp4 codes (one dword) -> 8 bf16 (an MFMA fragment), times `scale`
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t codes, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  return r;
}

// E8M0 byte -> 2^(b - 127) as fp32 (b = 0: 2^-127, a subnormal)
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) { return __uint_as_float(b ? (b << 23) : 0x00400000u); }

// waves that split one item's K: the fewest that fill the device's wave slots,
// up to `waves`
__device__ __forceinline__ int mx_waves_per_item(int64_t base, int64_t wave_slots, int waves, int nk) {
  int best = 1;
  for (int kw = 1; kw <= waves; kw *= 2) {
    if (kw > 1 && nk < kw * 2) break;
    best = kw;
    if (base * kw >= wave_slots) break;
  }
  return best;
}

}  // namespace

// out = act(A . dequant(W)) over the filled slots of the active experts; item =
// (active expert, 64-column block, m-chunk of MT*16 rows); KW waves of a
// workgroup split K (128-deep steps) and meet in LDS.
template <int MT, int WAVES, int STAGES>
__global__ __launch_bounds__(WAVES * 64, 2) void ffn_mx_stream(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Ws,
    uint16_t* __restrict__ out, const int32_t* __restrict__ kept_count, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, int N, int C, int K, int Ncols, int relu, int mch,
    const int32_t* __restrict__ gather, int64_t a_rows, ActiveFromKept afk) {
  __shared__ float red[WAVES * 4 * 4 * 64];
  __shared__ int s_act[1024];
  __shared__ int wsum[16];
  __shared__ double sl[16];
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int n_act;
  if (afk.kept != nullptr) {  // first GEMM of the token-order forward: the active list from the kept counts
    n_act = active_from_kept<WAVES * 64>(afk, N, s_act, wsum, sl);
    active = s_act;
  } else {
    n_act = n_active[0];
  }
  if (n_act > N) n_act = N;
  const int NCB = Ncols / 64;
  const int nk = K >> 7;  // 128-deep steps
  const int64_t base = (int64_t)n_act * NCB * mch;
  if (base <= 0) return;
  // one 16-row tile (decode-sized experts): at most 2 waves per item (the
  // 384-expert decode batch, 14 experts, C = 1: 94 -> 82 us per layer step
  // against 4; the LDS meeting of more partials costs more than the extra waves
  // give).  Larger tiles keep up to all 4 (the skewed 17-expert layer at C = 32
  // was 15% slower with 2)
  const int KW = mx_waves_per_item(base, (int64_t)gridDim.x * WAVES, MT == 1 && WAVES > 2 ? 2 : WAVES, nk);
  const int groups = WAVES / KW;
  const int g = w / KW, kw = w - g * KW;
  const int nx = (gridDim.x % kMxXcds == 0) ? kMxXcds : 1;
  const int xcd = blockIdx.x % nx;
  const int64_t slots_x = (int64_t)(gridDim.x / nx) * groups;
  const int64_t per_x = (base + nx - 1) / nx;
  const int64_t rounds = (per_x + slots_x - 1) / slots_x;
  const int myk = (nk - kw + KW - 1) / KW;  // my steps: kw, kw + KW, ...

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
    const int mtc = rows > 0 ? (rows + 15) >> 4 : 0;
    f32x4 acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (mtc > 0) {
      const int64_t ncb = (int64_t)e * Ncols;  // first column row of this expert
      const __amdgpu_buffer_rsrc_t qres = mx_rsrc(Wq + ncb * (K / 2), (int64_t)Ncols * (K / 2));
      const __amdgpu_buffer_rsrc_t sres = mx_rsrc(Ws + ncb * (K / 32), (int64_t)Ncols * (K / 32));
      const __amdgpu_buffer_rsrc_t ares = gather != nullptr
                                              ? mx_rsrc(A, a_rows * K * 2)
                                              : mx_rsrc(A + ((int64_t)e * C + m0) * K, (int64_t)rows * K * 2);
      int q_voff[4], s_voff[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = cb * 64 + 4 * c + j;  // lane c holds output columns 4c .. 4c+3
        q_voff[j] = n * (K / 2) + 16 * kg + kw * 64;
        s_voff[j] = n * (K / 32) + kw * 4;
      }
      int a_voff[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int rr = mt * 16 + c;
        const int64_t src = gather != nullptr && rr < rows ? gather[(int64_t)e * C + m0 + rr] : rr;
        a_voff[mt] = rr < rows ? (int)((src * K + kw * 128 + 32 * kg) * 2) : kMxOOR;
      }
      const int q_step = KW * 64, s_step = KW * 4, a_step = KW * 256;
      // one step's operands: the weight codes and scales and the token-row
      // fragments, loaded STAGES - 1 steps ahead together (the row fragments one
      // step ahead left each step waiting on its own row loads)
      struct WStage {
        u32x4 q[4];
        uint32_t s[4];
        u32x4 a[MT][4];
      };
      auto load_w = [&](WStage& d, int step) {
        const int st = step < myk ? step : myk - 1;  // past the end: re-read the last step (cache hit)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          d.q[j] = mx_load16(qres, q_voff[j], st * q_step);
          d.s[j] = mx_load4(sres, s_voff[j], st * s_step);
        }
      };
      const u32x4 zero = {0u, 0u, 0u, 0u};
      // padding steps (past myk) multiply a zero A fragment, selected where it is
      // used: a select right after the load would wait for the load at once
      auto load_a = [&](u32x4 (&d)[MT][4], int step) {
        const int st = step < myk ? step : myk - 1;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) d[mt][q] = mx_load16(ares, a_voff[mt], st * a_step + q * 16);
      };
      WStage ring[STAGES];
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s) {
        load_w(ring[s], s);
        load_a(ring[s].a, s);
      }
      const int nk_pad = (myk + STAGES - 1) / STAGES * STAGES;
      for (int it = 0; it < nk_pad; it += STAGES) {
#pragma unroll
        for (int u = 0; u < STAGES; ++u) {
          const int cur = it + u;
          load_w(ring[(u + STAGES - 1) % STAGES], cur + STAGES - 1);
          load_a(ring[(u + STAGES - 1) % STAGES].a, cur + STAGES - 1);
          __builtin_amdgcn_sched_barrier(0);
          const bool live = cur < myk;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // this lane's block: byte kg of the scale dword
            const float sc = e8m0_to_f32((ring[u].s[j] >> (8 * kg)) & 0xffu);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x4 bf = fp4x8_to_bf16(ring[u].q[j][q], sc);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                acc[mt][j] = mfma_bf16_16x16x32(live ? ring[u].a[mt][q] : zero, bf, acc[mt][j]);
            }
          }
        }
      }
    }

    auto store4 = [&](uint16_t* p, const float (&v)[4]) {
      float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
      if (relu) {
        a0 = fmaxf(a0, 0.f);
        a1 = fmaxf(a1, 0.f);
        a2 = fmaxf(a2, 0.f);
        a3 = fmaxf(a3, 0.f);
      }
      u32x2 o;
      o[0] = pack_bf2(a0, a1);
      o[1] = pack_bf2(a2, a3);
      *reinterpret_cast<u32x2*>(p) = o;
    };
    if (KW == 1) {
      if (mtc > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rl = mt * 16 + kg * 4 + i;
            if (mt < mtc && rl < rows) {
              float v[4] = {acc[mt][0][i], acc[mt][1][i], acc[mt][2][i], acc[mt][3][i]};
              store4(out + ((int64_t)e * C + m0 + rl) * Ncols + cb * 64 + c * 4, v);
            }
          }
      }
    } else {
      // the KW waves of a group sum their partials in LDS in wave order
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[((w * 4 + i) * 4 + j) * 64 + lane] = acc[mt][j][i];
        __syncthreads();
        if (mt < mtc) {
          for (int i = kw; i < 4; i += KW) {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float sum = 0.f;
              for (int q = 0; q < KW; ++q) sum += red[(((g * KW + q) * 4 + i) * 4 + j) * 64 + lane];
              v[j] = sum;
            }
            const int rl = mt * 16 + kg * 4 + i;
            if (rl < rows) store4(out + ((int64_t)e * C + m0 + rl) * Ncols + cb * 64 + c * 4, v);
          }
        }
        __syncthreads();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// quantizer: one thread per (expert, column n, 32-block b); consecutive threads
// take consecutive columns, so every load of the 32 block elements is coalesced
template <typename TW>
__global__ __launch_bounds__(256) void mx_quantize(const TW* __restrict__ w, int64_t batches, int K, int Ncols,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  const int64_t e = blockIdx.z;
  if (n >= Ncols) return;
  const TW* col = w + (e * K + (int64_t)b * 32) * Ncols + n;
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if constexpr (sizeof(TW) == 2) v[i] = bf2f(col[(int64_t)i * Ncols]);
    else v[i] = col[(int64_t)i * Ncols];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  // E = clamp(floor(log2 amax) - 2, -127, 127) from the bits (exact, subnormals included)
  int E = -127;
  if (amax > 0.f) {
    const uint32_t bits = __float_as_uint(amax);
    const int ex = (int)(bits >> 23);
    const int fl = ex > 0 ? ex - 127 : (31 - __clz((int)(bits & 0x7fffffu))) - 149;
    E = fl - 2;
    E = E < -127 ? -127 : (E > 127 ? 127 : E);
  }
  // 1 / 2^E as fp32: -E is in [-125, 127] here, a normal float
  const float inv = __uint_as_float((uint32_t)(127 - E) << 23);
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float r = v[i] * inv;
    const float a = fabsf(r);
    // nearest E2M1 magnitude, ties to the even mantissa: alternating > / >= at
    // the midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5; beyond 6 saturates
    const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    const uint32_t code = mag | ((__float_as_uint(v[i]) >> 28) & 8u);
    packed[i >> 3] |= code << (4 * (i & 7));
  }
  u32x4 o = {packed[0], packed[1], packed[2], packed[3]};
  *reinterpret_cast<u32x4*>(codes + ((e * Ncols + n) * (int64_t)(K / 2)) + b * 16) = o;
  scales[(e * Ncols + n) * (int64_t)(K / 32) + b] = (uint8_t)(E + 127);
}

// ---------------------------------------------------------------------------
static int mx_grid(const void* kernel, int threads) {
  int per_cu = 1, cus = 256, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1) per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  return per_cu * cus;
}

template <int MT>
static hipError_t launch_mx_mt(const void* A, const uint8_t* q, const uint8_t* s, void* out, const int32_t* kept,
                               const int32_t* active, const int32_t* n_active, int N, int C, int K, int Ncols,
                               int relu, hipStream_t st, const int32_t* gather, int64_t a_rows,
                               const ActiveFromKept& afk) {
  constexpr int kWaves = 4;
  constexpr int kStages = MT == 1 ? 4 : MT <= 2 ? 3 : 2;  // ring depth within the register budget
  auto kern = ffn_mx_stream<MT, kWaves, kStages>;
  const int mch = (C + MT * 16 - 1) / (MT * 16);
  const int grid = mx_grid(reinterpret_cast<const void*>(kern), kWaves * 64);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kWaves * 64), 0, st, static_cast<const uint16_t*>(A), q, s,
                     static_cast<uint16_t*>(out), kept, active, n_active, N, C, K, Ncols, relu, mch, gather, a_rows,
                     afk);
  return hipGetLastError();
}

bool mx_ffn_applies(int C, int d, int dff) { return C <= 64 && d % 128 == 0 && dff % 128 == 0; }

hipError_t launch_ffn_mx(const void* xin, const MxWeights& mw, int N, int C, int d, int dff,
                         const int32_t* kept_count, const int32_t* active, const int32_t* n_active, void* xout,
                         void* h, hipStream_t st, const int32_t* gather, int64_t a_rows, const ActiveFromKept& afk) {
  // up to 48 rows in one item; 49 .. 64 rows as two 32-row m-chunks (4 row tiles
  // of accumulators and A fragments would not fit in registers)
  const int mt = C <= 16 ? 1 : C <= 32 ? 2 : C <= 48 ? 3 : 2;
  auto one = [&](const void* A, const uint8_t* q, const uint8_t* s, void* o, int K, int Ncols, int relu,
                 const int32_t* ga, int64_t ar, const ActiveFromKept& ak) -> hipError_t {
    switch (mt) {
      case 1: return launch_mx_mt<1>(A, q, s, o, kept_count, active, n_active, N, C, K, Ncols, relu, st, ga, ar, ak);
      case 2: return launch_mx_mt<2>(A, q, s, o, kept_count, active, n_active, N, C, K, Ncols, relu, st, ga, ar, ak);
      default: return launch_mx_mt<3>(A, q, s, o, kept_count, active, n_active, N, C, K, Ncols, relu, st, ga, ar, ak);
    }
  };
  hipError_t e = one(xin, mw.w1_codes, mw.w1_scales, h, d, dff, 1, gather, a_rows, afk);
  if (e != hipSuccess) return e;
  return one(h, mw.w2_codes, mw.w2_scales, xout, dff, d, 0, nullptr, 0, ActiveFromKept{});
}

hipError_t launch_mx_quantize(const void* w, int dtype, int64_t batches, int K, int Ncols, uint8_t* codes,
                              uint8_t* scales, hipStream_t st) {
  dim3 grid((unsigned)((Ncols + 255) / 256), (unsigned)(K / 32), (unsigned)batches);
  if (dtype == 1)
    hipLaunchKernelGGL(mx_quantize<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(w), batches, K,
                       Ncols, codes, scales);
  else
    hipLaunchKernelGGL(mx_quantize<float>, grid, dim3(256), 0, st, static_cast<const float*>(w), batches, K, Ncols,
                       codes, scales);
  return hipGetLastError();
}

}  // namespace swm
