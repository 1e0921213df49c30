// bf16 x bf16 -> fp32 GEMM on gfx950 matrix cores, with the decode step's
// fused epilogues: C[m][n] = sum_k A[m][k] * B[n][k] (+ bias, then one of
// store fp32 / residual add / GELU to bf16 / Q-K-V scatter / pixel shuffle).
//
// Design (gfx950):
//  * v_mfma_f32_32x32x16_bf16; each wave owns a (TM*32) x (TN*32) sub-tile.
//  * A and B tiles of BK = 64 (128 bytes per row) are staged through LDS,
//    double-buffered, with one barrier per K step; the next K step's global
//    loads are issued before the current step's MFMAs.
//  * LDS rows are 8 chunks of 16 bytes; chunk c of row r is stored at
//    c ^ (r & 7), so the 8 consecutive rows read by 8 lanes for one MFMA
//    operand fall on 8 distinct bank groups.
//  * Tiles are dealt to the 8 XCDs in contiguous runs (workgroup i runs on
//    XCD i % 8), and inside a run in column-major groups of 8 tile rows, so
//    that the tiles resident on one XCD share A rows and B columns in its L2.
#include "fd_common.h"

namespace fd {
namespace {

constexpr int BK = 64;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

// Column-dependent part of an epilogue store, computed once per lane and
// 32-column block; the row-dependent part is added per element.
struct ColInfo {
  size_t base;   // element offset of row 0 of this column
  int kind;      // EPI_QKV: 0 = Q, 1 = K, 2 = V^T
  float bias;
};

template <int EPI>
__device__ __forceinline__ ColInfo col_info(const EpiParams& e, int n, int write_slot) {
  ColInfo ci;
  ci.bias = e.bias[n];
  ci.kind = 0;
  if constexpr (EPI == EPI_QKV) {
    const int D = e.d_model, hd = e.head_dim, heads = D / hd;
    const int which = n / D;
    const int r = n - which * D;
    const int head = r / hd, d = r - head * hd;
    ci.kind = which;
    if (which == 0)
      ci.base = (size_t)head * e.q_rows * hd + d;
    else if (which == 1)
      ci.base = ((size_t)write_slot * heads + head) * (size_t)e.n_pad * hd + d;
    else
      ci.base = ((size_t)write_slot * heads + head) * (size_t)hd * e.n_pad +
                (size_t)d * e.n_pad;
  } else if constexpr (EPI == EPI_PIXELS) {
    const int P = e.patch_out, C = e.out_c;
    const int per_t = P * P * C;
    const int tau = n / per_t;
    int r = n - tau * per_t;
    const int dy = r / (P * C);
    r -= dy * (P * C);                                   // dx * C + c
    ci.base = ((size_t)tau * e.pix_h + dy) * (size_t)e.pix_w * C + r;
  } else {
    ci.base = n;
  }
  return ci;
}

template <int EPI>
__device__ __forceinline__ void epi_store(const EpiParams& e, const ColInfo& ci,
                                          int m, float acc) {
  const float v = acc + ci.bias;
  if constexpr (EPI == EPI_F32_BIAS) {
    e.out_f32[ci.base + (size_t)m * e.ldo] = v;
  } else if constexpr (EPI == EPI_RESID) {
    float* p = e.out_f32 + ci.base + (size_t)m * e.ldo;
    *p = *p + v;
  } else if constexpr (EPI == EPI_GELU_BF16) {
    e.out_bf16[ci.base + (size_t)m * e.ldo] = f2bf(gelu_erf(v));
  } else if constexpr (EPI == EPI_QKV) {
    if (ci.kind == 0)
      e.out_bf16[ci.base + (size_t)m * e.head_dim] = f2bf(v * e.q_scale);
    else if (ci.kind == 1)
      e.ring_k[ci.base + (size_t)m * e.head_dim] = f2bf(v);
    else
      e.ring_vt[ci.base + vt_perm(m)] = f2bf(v);
  } else if constexpr (EPI == EPI_PIXELS) {
    // token m = (i, j) -> pixel row i*P, column j*P
    const int i = m / e.tok_w, j = m - i * e.tok_w;
    const size_t row = ((size_t)i * e.patch_out * e.pix_w + (size_t)j * e.patch_out) * e.out_c;
    e.out_f32[ci.base + row] = v;
  }
}

// Block tile BM x BN, waves WAVES_M x WAVES_N; each wave (BM/WAVES_M) x (BN/WAVES_N).
template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI>
__global__ __launch_bounds__(kWave * WAVES_M * WAVES_N)
void gemm_bf16_kernel(const GemmArgs args_in) {
  const GemmArgs args = args_in;
  constexpr int NT = kWave * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int ROWS = BM + BN;               // LDS rows per stage
  constexpr int CHUNKS = ROWS * 8;            // 16-byte chunks per stage
  static_assert(CHUNKS % NT == 0, "tile chunks must divide evenly");
  constexpr int CPT = CHUNKS / NT;            // chunks per thread
  constexpr int STAGE = ROWS * 128;           // bytes per stage
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int K = args.k;
  const int tiles_m = (args.m + BM - 1) / BM;
  const int tiles_n = args.n / BN;
  const int T = tiles_m * tiles_n;

  // XCD-aware remap: the run of logical tiles [x*per + min(x,rem), ...) goes
  // to XCD x.
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds, idx = bid / kXcds;
  const int per = T / kXcds, rem = T % kXcds;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + idx;
  // Column-major inside groups of 8 tile rows.
  constexpr int GM = 8;
  const int group = logical / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int in_g = logical - group * GM * tiles_n;
  const int tm = first_m + in_g % gsize;
  const int tn = in_g / gsize;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;

  const uint16_t* gA = args.a + (size_t)tm * BM * K;
  const uint16_t* gB = args.b + (size_t)tn * BN * K;

  // Per-thread global source and LDS destination of its chunks.
  const uint16_t* src[CPT];
  int dst[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int q = tid + i * NT;
    const int row = q >> 3, c = q & 7;
    src[i] = (row < BM ? gA + (size_t)row * K : gB + (size_t)(row - BM) * K) + c * 8;
    dst[i] = swz(row, c);
  }

  uint4 stage_regs[CPT];
#define FD_GEMM_GLOAD(KT_)                                                   \
  _Pragma("unroll") for (int i_ = 0; i_ < CPT; ++i_)                        \
    stage_regs[i_] = *reinterpret_cast<const uint4*>(src[i_] + (KT_) * BK);
#define FD_GEMM_LSTORE(BUF_)                                                 \
  _Pragma("unroll") for (int i_ = 0; i_ < CPT; ++i_)                        \
    *reinterpret_cast<uint4*>(smem + (BUF_) * STAGE + dst[i_]) = stage_regs[i_];

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int KT = K / BK;
  FD_GEMM_GLOAD(0)
  FD_GEMM_LSTORE(0)
  __syncthreads();

  const int r32 = lane & 31, half = lane >> 5;
  // One K step of MFMAs on LDS stage BUF_.
#define FD_GEMM_COMPUTE(BUF_)                                                   \
  {                                                                             \
    const uint8_t* sA = smem + (BUF_) * STAGE;                                  \
    const uint8_t* sB = sA + BM * 128;                                          \
    _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                          \
      const int chunk = kk * 2 + half;                                          \
      bf16x8 af[TM], bfr[TN];                                                   \
      _Pragma("unroll") for (int i = 0; i < TM; ++i) af[i] =                    \
          *reinterpret_cast<const bf16x8*>(sA + swz(wm * WM + i * 32 + r32, chunk)); \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) bfr[j] =                   \
          *reinterpret_cast<const bf16x8*>(sB + swz(wn * WN + j * 32 + r32, chunk)); \
      _Pragma("unroll") for (int i = 0; i < TM; ++i)                            \
      _Pragma("unroll") for (int j = 0; j < TN; ++j)                            \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j],    \
                                                              acc[i][j], 0, 0, 0); \
    }                                                                           \
  }
  // Steady state: fetch step kt+1 to registers, compute step kt, park the
  // fetched step in the other LDS stage, one barrier.  Last step peeled.
  for (int kt = 0; kt + 1 < KT; ++kt) {
    FD_GEMM_GLOAD(kt + 1)
    FD_GEMM_COMPUTE(kt & 1)
    FD_GEMM_LSTORE((kt + 1) & 1)
    __syncthreads();
  }
  FD_GEMM_COMPUTE((KT - 1) & 1)
#undef FD_GEMM_COMPUTE

#undef FD_GEMM_GLOAD
#undef FD_GEMM_LSTORE
  const EpiParams epi = args.epi;
  int write_slot = 0;
  if constexpr (EPI == EPI_QKV) write_slot = epi.state->write_slot;

  // Accumulator layout of a 32x32 block: column = lane % 32,
  // row = 8 * (v / 4) + 4 * (lane / 32) + v % 4.
  const int m0 = tm * BM + wm * WM;
  const int n0 = tn * BN + wn * WN;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const ColInfo ci = col_info<EPI>(epi, n0 + j * 32 + r32, write_slot);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (m < args.m) epi_store<EPI>(epi, ci, m, acc[i][j][v]);
      }
  }
}

template <int BM, int BN, int WM_, int WN_>
hipError_t launch_epi(int epi, const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.m + BM - 1) / BM) * (a.n / BN);
  dim3 grid(tiles), block(kWave * WM_ * WN_);
  switch (epi) {
    case EPI_F32_BIAS:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM_, WN_, EPI_F32_BIAS>), grid, block, 0, s, a);
      break;
    case EPI_RESID:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM_, WN_, EPI_RESID>), grid, block, 0, s, a);
      break;
    case EPI_GELU_BF16:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM_, WN_, EPI_GELU_BF16>), grid, block, 0, s, a);
      break;
    case EPI_QKV:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM_, WN_, EPI_QKV>), grid, block, 0, s, a);
      break;
    case EPI_PIXELS:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM_, WN_, EPI_PIXELS>), grid, block, 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Pick a tile: 256x256 (8 waves of 128x64) when the problem yields at least
// one full wave of tiles on 256 CUs, else 128x128 (4 waves of 64x64), else
// 64x64 (4 waves of 32x32).  m_rows_alloc (rows of A) must be a multiple of
// the chosen BM; callers allocate activations in multiples of 256 rows.
hipError_t launch_gemm(int epi, const GemmArgs& a, int m_rows_alloc, hipStream_t s) {
  if (a.n <= 0 || a.k <= 0 || a.k % BK != 0) return hipErrorInvalidValue;
  if (a.m <= 0) return hipSuccess;
  const long big_tiles = (long)((a.m + 255) / 256) * (a.n / 256);
  if (a.n % 256 == 0 && m_rows_alloc % 256 == 0 && big_tiles >= 192)
    return launch_epi<256, 256, 2, 4>(epi, a, s);
  if (a.n % 128 == 0 && m_rows_alloc % 128 == 0 &&
      (long)((a.m + 127) / 128) * (a.n / 128) >= 128)
    return launch_epi<128, 128, 2, 2>(epi, a, s);
  if (a.n % 64 == 0 && m_rows_alloc % 64 == 0)
    return launch_epi<64, 64, 2, 2>(epi, a, s);
  return hipErrorInvalidValue;
}

}  // namespace fd
