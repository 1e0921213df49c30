// HBM-bound steps of the decode: LayerNorm, patchify, ring bookkeeping.
//
// [FD] = "FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder with
// Transformers" (academ.us/article/2607.14898).
#include "fd_common.h"

namespace fd {
namespace {

// DPP move of src with control CTRL into the lanes of the rows in ROW_MASK
// (other lanes read 0).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp0(float src) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(src), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the wave, returned to every lane.  DPP adds instead of LDS
// permutes: quad_perm [1,0,3,2] and [2,3,0,1] sum each group of 4 lanes,
// row_half_mirror and row_mirror each row of 16; row_bcast:15 (into rows 1
// and 3) and row_bcast:31 (into rows 2 and 3) carry the row sums up to lane
// 63, which is read back as a scalar.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp0<0xB1>(v);
  v += dpp0<0x4E>(v);
  v += dpp0<0x141>(v);
  v += dpp0<0x140>(v);
  v += dpp0<0x142, 0xA>(v);
  v += dpp0<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Pre-sublayer norm ([FD] §3.2 "Base Architecture").  LayerNorm:
// y = (x - mean) / sqrt(biased var + eps) * g + b; with RMS (the paper's
// RMSNorm): y = x / sqrt(mean(x^2) + eps) * g.  Statistics in fp32, output
// rounded to bf16 as the next GEMM's A operand.  One wave per row; a lane
// keeps its E = d / 64 values (float4-strided when d % 256 == 0) in registers
// so the row is read from HBM once.
template <int E, bool RMS>
__global__ __launch_bounds__(256)
void layernorm_kernel(const float* __restrict__ h, int m, int d,
                      const float* __restrict__ g, const float* __restrict__ b,
                      float eps, uint16_t* __restrict__ out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= m) return;
  const float* x = h + (size_t)row * d;
  float v[E];
  if constexpr (E % 4 == 0) {
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const float4 t = *reinterpret_cast<const float4*>(x + i * 256 + lane * 4);
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = x[i * 64 + lane];
  }
  float mean = 0.0f;
  if constexpr (!RMS) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) s += v[i];
    mean = wave_sum(s) * (1.0f / (float)d);
  }
  float q = 0.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const float c = v[i] - mean;
    q += c * c;
  }
  const float rstd = rsqrtf(wave_sum(q) * (1.0f / (float)d) + eps);
  uint16_t* y = out + (size_t)row * d;
  if constexpr (E % 4 == 0) {
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const int col = i * 256 + lane * 4;
      const float4 gg = *reinterpret_cast<const float4*>(g + col);
      const float4 bb = RMS ? make_float4(0.0f, 0.0f, 0.0f, 0.0f)
                            : *reinterpret_cast<const float4*>(b + col);
      uint2 w;
      w.x = f2bf2((v[4 * i] - mean) * rstd * gg.x + bb.x,
                  (v[4 * i + 1] - mean) * rstd * gg.y + bb.y);
      w.y = f2bf2((v[4 * i + 2] - mean) * rstd * gg.z + bb.z,
                  (v[4 * i + 3] - mean) * rstd * gg.w + bb.w);
      *reinterpret_cast<uint2*>(y + col) = w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int col = i * 64 + lane;
      y[col] = f2bf((v[i] - mean) * rstd * g[col] + (RMS ? 0.0f : b[col]));
    }
  }
}

// Tokens of one latent frame ([FD] §3.2 Eq. 1: raster order; §4.3: p x p
// PixelUnshuffle fold).  x[n][f], n = i*(wl/p) + j, f = c*p*p + dy*p + dx,
// = bf16(z[c][i*p+dy][j*p+dx]); features f >= c*p*p (K padding) are 0.
// A workgroup covers kPatchTJ consecutive tokens of token row i and moves
// kPatchFC features at a time through LDS: the reads run along latent rows
// (the tokens' columns j*p + dx are contiguous) and the writes along token
// rows, so both are contiguous.  P is a template argument so that each
// thread's loads are unrolled and in flight together.
constexpr int kPatchTJ = 32, kPatchFC = 64;
template <int P>
__global__ __launch_bounds__(256)
void patchify_kernel(const float* __restrict__ z_arg, const DeviceState* __restrict__ io,
                     size_t z_off, int c, int hl, int wl, int k_pad,
                     uint16_t* __restrict__ x) {
  // With io the latent is the frame's buffer recorded in the ring state.
  const float* __restrict__ z = io ? io->latent + z_off : z_arg;
  __shared__ float tile[kPatchFC][kPatchTJ + 1];
  constexpr int PP = P * P;
  constexpr int ROWS = kPatchFC / P;           // (channel, dy) pairs of a feature block
  constexpr int COLS = kPatchTJ * P;           // latent columns of the tokens
  static_assert(kPatchFC % PP == 0 && (ROWS * COLS) % 256 == 0, "patchify tiling");
  const int tw = wl / P;
  const int i = blockIdx.y, j0 = blockIdx.x * kPatchTJ;
  const int nj = min(kPatchTJ, tw - j0);
  const int nf = c * PP;
  for (int f0 = 0; f0 < k_pad; f0 += kPatchFC) {
    float v[ROWS * COLS / 256];
#pragma unroll
    for (int u = 0; u < ROWS * COLS / 256; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int r = e / COLS, col = e - r * COLS;
      const int chl = r / P, dy = r - chl * P;
      const int jj = col / P, dx = col - jj * P;
      const int f = f0 + chl * PP + dy * P + dx;
      v[u] = jj < nj && f < nf
                 ? z[((size_t)(f / PP) * hl + i * P + dy) * wl + (size_t)(j0 + jj) * P + dx]
                 : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < ROWS * COLS / 256; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int r = e / COLS, col = e - r * COLS;
      const int chl = r / P, dy = r - chl * P;
      const int jj = col / P, dx = col - jj * P;
      tile[chl * PP + dy * P + dx][jj] = v[u];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPatchTJ * (kPatchFC / 2) / 256; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int jj = e / (kPatchFC / 2), fp = e - jj * (kPatchFC / 2);
      if (jj < nj)
        *reinterpret_cast<uint32_t*>(x + (size_t)(i * tw + j0 + jj) * k_pad + f0 + 2 * fp) =
            f2bf2(tile[2 * fp][jj], tile[2 * fp + 1][jj]);
    }
    __syncthreads();
  }
}

// Start of a frame ([FD] §3.3 Eq. 2): frame t takes slot t mod W, which held
// frame t - W (evicted); the valid frames are max(0, t-W+1) .. t.
__global__ void frame_begin_kernel(DeviceState* st, int window) {
  if (threadIdx.x != 0) return;
  const int t = st->frames_done;
  const int slot = t % window;
  const int nv = (t + 1) < window ? (t + 1) : window;
  st->t = t;
  st->write_slot = slot;
  st->n_valid = nv;
  st->slot_frame[slot] = t;
  for (int i = 0; i < FD_MAX_WINDOW; ++i)
    st->chrono_slot[i] = i < nv ? (t - nv + 1 + i) % window : 0;
  st->frames_done = t + 1;
}

// Store one frame's temporal rotary table (kernel argument) into device
// memory; every index is a compile-time constant, so the argument is read
// straight from the kernel-argument segment.
__global__ void rope_table_kernel(float2* dst, const RopeTable tab) {
  if (threadIdx.x != 0) return;
#pragma unroll
  for (int r = 0; r < kRopeRows; ++r)
#pragma unroll
    for (int k = 0; k < 12; ++k) dst[r * 12 + k] = tab.v[r][k];
}

// Test support: bf16 NaN into the token rows of every ring slot (K rows
// t < n, V^T columns vt_perm(t) for t < n; vt_perm is its own inverse), so that
// a read of a slot no frame has written shows up as NaN pixels.
__global__ __launch_bounds__(256)
void poison_ring_kernel(uint16_t* __restrict__ ring_k, uint16_t* __restrict__ ring_vt,
                        long total, int n, int n_pad, int hd) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int kt = (int)((idx / hd) % n_pad);       // K: token of [head][n_pad][hd]
  const int vc = (int)(idx % n_pad);              // V^T: column of [head][hd][n_pad]
  if (kt < n) ring_k[idx] = 0x7FC0;
  if (vt_perm(vc) < n) ring_vt[idx] = 0x7FC0;
}

__global__ void state_reset_kernel(DeviceState* st) {
  if (threadIdx.x != 0) return;
  st->frames_done = 0;
  st->t = 0;
  st->write_slot = 0;
  st->n_valid = 0;
  for (int i = 0; i < FD_MAX_WINDOW; ++i) {
    st->slot_frame[i] = -1;
    st->chrono_slot[i] = 0;
  }
  st->latent = nullptr;
  st->pixels = nullptr;
}

}  // namespace

hipError_t launch_layernorm(const float* h, int m, int d, const float* g,
                            const float* b, float eps, int rms, uint16_t* out,
                            hipStream_t s) {
  if (m <= 0) return hipSuccess;
  dim3 grid((m + 3) / 4), block(256);
  switch (d) {
#define FD_LN_CASE(D_)                                                      \
    case D_:                                                                \
      if (rms)                                                              \
        hipLaunchKernelGGL((layernorm_kernel<D_ / 64, true>), grid, block, 0, s, \
                           h, m, d, g, b, eps, out);                        \
      else                                                                  \
        hipLaunchKernelGGL((layernorm_kernel<D_ / 64, false>), grid, block, 0, s, \
                           h, m, d, g, b, eps, out);                        \
      break;
    FD_LN_CASE(64) FD_LN_CASE(128) FD_LN_CASE(192) FD_LN_CASE(256)
    FD_LN_CASE(384) FD_LN_CASE(512) FD_LN_CASE(768) FD_LN_CASE(1024)
    FD_LN_CASE(1536) FD_LN_CASE(2048)
#undef FD_LN_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_patchify(const float* z, const DeviceState* io, size_t z_off, int c, int hl,
                           int wl, int p, int k_pad, uint16_t* x, hipStream_t s) {
  const int th = hl / p, tw = wl / p;
  if (th <= 0 || tw <= 0 || k_pad <= 0) return hipSuccess;
  // Feature blocks of kPatchFC cover the padded feature count.
  if (k_pad % kPatchFC || (p != 1 && p != 2)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((tw + kPatchTJ - 1) / kPatchTJ), th);
  if (p == 1)
    hipLaunchKernelGGL(patchify_kernel<1>, grid, dim3(256), 0, s, z, io, z_off, c, hl, wl, k_pad,
                       x);
  else
    hipLaunchKernelGGL(patchify_kernel<2>, grid, dim3(256), 0, s, z, io, z_off, c, hl, wl, k_pad,
                       x);
  return hipGetLastError();
}

// Record the caller's buffers of the next frame in the ring state.
__global__ void set_io_kernel(DeviceState* st, const float* latent, float* pixels) {
  if (threadIdx.x != 0) return;
  st->latent = latent;
  st->pixels = pixels;
}

hipError_t launch_set_io(DeviceState* st, const float* latent, float* pixels, hipStream_t s) {
  hipLaunchKernelGGL(set_io_kernel, dim3(1), dim3(64), 0, s, st, latent, pixels);
  return hipGetLastError();
}

hipError_t launch_frame_begin(DeviceState* st, int window, hipStream_t s) {
  hipLaunchKernelGGL(frame_begin_kernel, dim3(1), dim3(64), 0, s, st, window);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* dst, const RopeTable& tab, hipStream_t s) {
  hipLaunchKernelGGL(rope_table_kernel, dim3(1), dim3(64), 0, s, dst, tab);
  return hipGetLastError();
}

hipError_t launch_poison_ring(uint16_t* ring_k, uint16_t* ring_vt, int heads, int n,
                              int n_pad, int hd, hipStream_t s) {
  const long total = (long)heads * n_pad * hd;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(poison_ring_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     ring_k, ring_vt, total, n, n_pad, hd);
  return hipGetLastError();
}

hipError_t launch_state_reset(DeviceState* st, hipStream_t s) {
  hipLaunchKernelGGL(state_reset_kernel, dim3(1), dim3(64), 0, s, st);
  return hipGetLastError();
}

}  // namespace fd
