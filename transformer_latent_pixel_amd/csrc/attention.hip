// Mask-free attention of one frame's queries over the rolling K/V ring.
//
// Operation ([FD] = "FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder
// with Transformers", academ.us/article/2607.14898, §3.3 "Frame-by-Frame
// Processing" step (3) and "Attention Pattern"): per head, the N queries of
// frame t attend to every key of the n_valid cached frames (t-n_valid+1 .. t,
// oldest first), O = softmax(Q K^T / sqrt(hd)) V, with no mask.  The scale
// and log2(e) are folded into Q by the QKV epilogue, so scores come out in
// log2 units and the softmax uses exp2.
//
// gfx950 design (head_dim 64):
//  * A workgroup is one head x 512 queries (8 waves x 64); when that leaves
//    CUs idle, the cached key tiles are split over 2-4 workgroups and a
//    second kernel merges their partial outputs.  Keys are streamed in tiles
//    of 64 through a 4-stage LDS ring filled by direct global->LDS loads
//    ahead of use: a K tile [key][d] and a V^T tile [d][key], 128-byte rows,
//    16-byte chunks XOR-swizzled by row pairs.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16
//    with Q held in registers.  A lane then owns one query column and 16 keys
//    of each 32x32 block, so row max and row sum are in-lane plus one
//    exchange with the lane 32 away.
//  * The running max is subtracted by the MFMA itself: a fifth k-chunk pairs
//    a K-side row (1, mask) with a Q-side column (-max, 1), which also puts
//    -1e30 on the padded keys of a frame's last tile.  The max is lazy: it
//    starts at 0 and stays there while scores stay within 2^64 of it (the
//    chunk is then needed only on ragged tiles); the common path computes no
//    tile max at all.  The key tiles are first run with no check inside the
//    loop (the per-tile branch would end the loop body's basic block and
//    cost about 7% of its cycles), with the row sums accumulated by a
//    16x16x32 MFMA rather than VALU dot products (which barely overlap the
//    other wave's MFMAs).  If a row sum ended above 2^64 (any weight above
//    2^64 implies that), the whole workgroup runs its tiles again with the
//    per-tile check, which moves the max and recomputes that tile's
//    weights, and sums by v_dot2.  Both runs add the same bf16 weights in
//    fp32, in different orders.
//  * Online softmax (running max and sum per query, fp32).  P^T, rounded to
//    bf16, is already laid out as the B operand of O^T = V^T P^T: the ring
//    stores V transposed with key bits 2 and 3 swapped inside 32-key groups
//    (vt_perm), so each lane's 8 keys of a 16-key chunk are one 16-byte read.
//  * Workgroups are dealt to XCDs in contiguous (head, query-tile) runs, so
//    the workgroups sharing a head's K/V sit on one XCD's L2.
#include <math.h>

#include <mutex>

#include "fd_common.h"
#include "flashdec_kernels.h"

// Scratch of fdk_attention_noalloc, for callers that cannot allocate: the
// ring, the padded queries, the ring state and the key-split partials of one
// call.  Every GPU the library runs on holds its own copy until the process
// ends.  In host code the name is only a stand-in for the symbol: the device
// address comes from hipGetSymbolAddress (see noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[FDK_NOALLOC_SCRATCH_BYTES];

namespace fd {
namespace {

// LDS tile layout: 64 rows of 128 bytes (8 chunks of 16 bytes); chunk c of
// row r sits at c ^ ((r >> 1) & 7).  A 16-byte LDS read serves 16 lanes per
// cycle over 16 groups of 16 bytes; the 16 consecutive rows those lanes read
// at one chunk (rows of one parity share (8 r) mod 16) fall on 16 distinct
// groups.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

constexpr int AK = 64;    // keys per tile

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Barrier that orders waves without draining loads still in flight (each
// wave has already waited for its own loads of the stage it will read).
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global -> LDS load of 16 bytes per lane (lane i lands at lds +
// 16 i): global_load_lds_dwordx4 with a wave-uniform 64-bit base, a per-lane
// 32-bit offset and the LDS destination in M0, written out so that the
// compiler does not track it.  Tracked, it makes the compiler put a wait for
// every load in flight (the refill just issued included) before some steps'
// LDS reads: it cannot always tell that they read another stage.  The ring's
// own vmcnt waits and barriers order these loads.  The instruction writes no
// register and reads its address operands at issue; M0 is not used by any
// other instruction of this file's kernels.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, const void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(m0)
               : "memory");
}

__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

// NW waves of 64 queries per workgroup; STAGES-deep LDS ring (3 or 4).  All
// waves meet the per-tile barrier at the same point (a schedule that offsets
// the two waves of a SIMD by half a tile measured slower).
template <int NW, int STAGES>
__global__ __launch_bounds__(NW * 64, 8 / NW)
void attention_hd64_kernel(const AttnArgs args_in) {
  const AttnArgs args = args_in;
  constexpr int HD = 64;
  constexpr int QPW = NW * 64;                 // queries per workgroup
  constexpr int TILE = AK * 128;               // bytes of one K or V^T tile
  constexpr int LPW = 16 / NW;                 // 1-KB loads per wave per tile
  static_assert(STAGES == 3 || STAGES == 4, "ring depth");
  // Ring of K and V^T tiles, one LDS object per stage and tensor.
  __shared__ __attribute__((aligned(1024))) uint8_t sk0[TILE], sv0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sk1[TILE], sv1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sk2[TILE], sv2[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sk3[STAGES == 4 ? TILE : 16],
      sv3[STAGES == 4 ? TILE : 16];
  __shared__ int rerun;                        // some wave's weights passed 2^64

  const int n = args.n, n_pad = args.n_pad, heads = args.heads;
  const int splits = args.splits;
  const int qtiles = (n + QPW - 1) / QPW;
  const int T = heads * qtiles * splits;
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds, idx = bid / kXcds;
  const int per = T / kXcds, rem = T % kXcds;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + idx;
  const int split = logical % splits;
  const int hq = logical / splits;
  const int head = hq / qtiles;
  const int q0 = (hq - head * qtiles) * QPW;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid == 0) rerun = 0;
  const int r32 = lane & 31, half = lane >> 5;

  const DeviceState* st = args.state;
  const int n_valid = st->n_valid;
  int chrono[FD_MAX_WINDOW];
#pragma unroll
  for (int i = 0; i < FD_MAX_WINDOW; ++i) chrono[i] = st->chrono_slot[i];

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[q][kk*16 + half*8 .. +8].
  bf16x8 qf[2][4];
  {
    const uint16_t* qbase = args.q + ((size_t)head * args.q_rows + q0 + wave * 64) * HD;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qf[qb][kk] = *reinterpret_cast<const bf16x8*>(
            qbase + (size_t)(qb * 32 + r32) * HD + kk * 16 + half * 8);
    // Let the Q loads land before the first refill: otherwise the compiler,
    // unsure at the loop head whether they have, puts a wait for every load
    // in flight (the refill just issued included) into the first step of
    // every unrolled loop iteration.
    wait_vmcnt<0>();
  }

  // A fifth k-chunk appended to S^T = K Q^T: K side row (1, mask_key, 0...),
  // Q side column (-mrun_q, 1, 0...), so the MFMA itself adds -mrun_q to
  // every score and -1e30 to keys past n (the padded end of a frame's last
  // tile).  Only lanes of the first half-wave carry k = 0, 1 of the chunk.
  bf16x8 kext_full, kext_tail[2], mext[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    kext_full[j] = to_bf16(0.0f);
    kext_tail[0][j] = to_bf16(0.0f);
    kext_tail[1][j] = to_bf16(0.0f);
    mext[0][j] = to_bf16(0.0f);
    mext[1][j] = to_bf16(0.0f);
  }
  const int tps = n_pad / AK;                  // tiles per cached frame
  const int tail_key0 = (tps - 1) * AK;
  if (half == 0) {
    kext_full[0] = to_bf16(1.0f);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      kext_tail[kb][0] = to_bf16(1.0f);
      kext_tail[kb][1] = to_bf16(tail_key0 + kb * 32 + r32 < n ? 0.0f : -1e30f);
    }
    mext[0][1] = to_bf16(1.0f);
    mext[1][1] = to_bf16(1.0f);
  }
  const bool tail_masked = (n % AK) != 0;

  // DMA plan: per tile 8 K loads + 8 V^T loads of 1 KB (8 rows of 128 bytes),
  // LPW per wave: wave w moves K rows and V^T rows w*(64/NW) ..  Lane i of a
  // load lands on row row0 + i/8, physical chunk i%8, so it fetches logical
  // chunk (i%8) ^ ((row >> 1) & 7) of that row.
  uint32_t voff[LPW];
  int lds_row0[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int row0 = wave * (64 / NW) + (j % (LPW / 2)) * 8;
    const int row = row0 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    lds_row0[j] = row0 * 128;
    voff[j] = j < LPW / 2 ? (uint32_t)(row * 128 + c * 16)
                          : (uint32_t)(row * n_pad * 2 + c * 16);
  }
  // Grouped-query attention: this query head reads KV head kvh of the ring.
  const int kvh = head * args.kv_heads / heads;
  const size_t slot_bytes = (size_t)args.kv_heads * n_pad * HD * 2;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(args.ring_k) +
                         (size_t)kvh * n_pad * HD * 2;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(args.ring_vt) +
                         (size_t)kvh * HD * n_pad * 2;
  // This split's key tiles, in chronological order over the cached frames:
  // [t0, t1) of the n_valid * tps tiles (possibly empty for tiny inputs).
  const int ntiles_all = n_valid * tps;
  const int t0 = (int)((long)split * ntiles_all / splits);
  const int t1 = (int)((long)(split + 1) * ntiles_all / splits);
  const int ntiles = t1 - t0;
  // Next tile to fetch, as (frame, first key, slot offset), advanced by one
  // tile per fetch and held at the split's last tile once every tile has been
  // issued (the extra fetches repeat it, keeping every wave's count of loads
  // in flight the same).
  int iss_t = t0, iss_f = 0, iss_key0 = 0;
  size_t iss_sb = 0;
  if (ntiles > 0) {
    iss_f = t0 / tps;
    iss_key0 = (t0 - iss_f * tps) * AK;
    int slot0 = chrono[0];
#pragma unroll
    for (int i = 1; i < FD_MAX_WINDOW; ++i)
      if (iss_f == i) slot0 = chrono[i];
    iss_sb = (size_t)slot0 * slot_bytes;
  }
  const int iss_f0 = iss_f, iss_key00 = iss_key0;
  const size_t iss_sb0 = iss_sb;

#define FD_ATT_ISSUE(SK_, SV_)                                                      \
  {                                                                                 \
    const uint8_t* kb_ = kbase + iss_sb + (size_t)iss_key0 * HD * 2;                \
    const uint8_t* vb_ = vbase + iss_sb + (size_t)iss_key0 * 2;                     \
    _Pragma("unroll") for (int j_ = 0; j_ < LPW; ++j_) {                           \
      asm volatile("" : "+v"(voff[j_]));                                            \
      const bool isk_ = j_ < LPW / 2;                                               \
      dma16(isk_ ? kb_ : vb_, voff[j_], (isk_ ? (SK_) : (SV_)) + lds_row0[j_]);     \
    }                                                                               \
    if (iss_t + 1 < t1) {                                                           \
      ++iss_t;                                                                      \
      iss_key0 += AK;                                                               \
      if (iss_key0 == tps * AK) {                                                   \
        iss_key0 = 0;                                                               \
        ++iss_f;                                                                    \
        int slot_ = chrono[0];                                                      \
        _Pragma("unroll") for (int i_ = 1; i_ < FD_MAX_WINDOW; ++i_)               \
          if (iss_f == i_) slot_ = chrono[i_];                                      \
        iss_sb = (size_t)slot_ * slot_bytes;                                        \
      }                                                                             \
    }                                                                               \
  }

  floatx16 o[2][2];                            // O^T blocks [d-block][q-block]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[a][b][v] = 0.0f;
  // Softmax state per query column, identical in both half-waves.  mrun is a
  // bf16 value (it enters the MFMA); scores are kept relative to it (log2
  // units).  It starts at 0 and stays there unless the first tile's max lies
  // outside [-kHome, kHome]; later it only moves when a weight
  // p = 2^(s - mrun) could exceed 2^kLazy (see FD_ATT_PV).  Weights up to
  // 2^64 are exact bf16 values and their sums stay far inside fp32 range.
  // While mrun is 0 for every column of a wave, the fifth k-chunk (which
  // subtracts mrun) is skipped except on a frame's ragged last tile (which
  // it masks).
  constexpr float kHome = 64.0f;
  constexpr float kLazySum = 18446744073709551616.0f;   // 2^64
  float mrun[2] = {0.0f, 0.0f};
  bool ext_on = false;                         // some column of the wave has mrun != 0
  float lrun[2] = {0.0f, 0.0f};                // this half-wave's partial sums
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  // Unchecked run: row sums by v_mfma_f32_16x16x32_bf16 with P^T fragment
  // pb[c][qb] as the B operand (lane i gives 8 keys of query column i % 32)
  // and a 0/1 A operand whose row 0 takes lanes 0 and 32 and row 1 lanes 17
  // and 49.  Row 0 of the 16x16 result then sums query column n = lane % 16
  // over lanes n and n + 32, row 1 column n + 16 over lanes n + 16 and n + 48:
  // lane n (< 16) holds the sums of queries n and n + 16 in elements 0 and 1.
  floatx4 lsum[2];
  bf16x8 sel16;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    sel16[j] = to_bf16(lane == 0 || lane == 32 || lane == 17 || lane == 49 ? 1.0f : 0.0f);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int v = 0; v < 4; ++v) lsum[a][v] = 0.0f;

  // Scores of one 64-key tile from K stage SK_ into s, relative to the
  // running max (log2 units), padded keys at -1e30.
#define FD_ATT_QK(SK_, TILE_)                                                        \
  {                                                                                  \
    const int tile_ = (TILE_);                                                       \
    const bool masked_ = tail_masked && (tile_ % tps) == tps - 1;                    \
    _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                 \
    _Pragma("unroll") for (int qb = 0; qb < 2; ++qb)                                 \
    _Pragma("unroll") for (int v = 0; v < 16; ++v) s[kb][qb][v] = 0.0f;              \
    _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                               \
      bf16x8 kf[2];                                                                  \
      _Pragma("unroll") for (int kb = 0; kb < 2; ++kb) kf[kb] =                      \
          *reinterpret_cast<const bf16x8*>((SK_) + swz(kb * 32 + r32, kk * 2 + half)); \
      _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                               \
      _Pragma("unroll") for (int qb = 0; qb < 2; ++qb)                               \
        s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb], qf[qb][kk],      \
                                                            s[kb][qb], 0, 0, 0);     \
    }                                                                                \
    if (ext_on || masked_) {                                                         \
      _Pragma("unroll") for (int kb = 0; kb < 2; ++kb) {                             \
        const bf16x8 ke_ = masked_ ? kext_tail[kb] : kext_full;                      \
        _Pragma("unroll") for (int qb = 0; qb < 2; ++qb)                             \
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ke_, mext[qb],         \
                                                              s[kb][qb], 0, 0, 0);   \
      }                                                                              \
    }                                                                                \
  }

  // P^T = 2^s rounded to bf16, laid out as the B operand of O^T += V^T P^T,
  // and with SUM_ this lane's partial row sums TS_ over its 32 keys of the
  // tile (the same bf16 values, added by v_dot2 against (1, 1)).
#define FD_ATT_EXP(TS_, SUM_)                                                        \
  _Pragma("unroll") for (int qb = 0; qb < 2; ++qb) {                                 \
    float ls = 0.0f;                                                                 \
    _Pragma("unroll") for (int c = 0; c < 4; ++c) {                                  \
      _Pragma("unroll") for (int j = 0; j < 8; j += 2) {                             \
        bf16x2 pr;                                                                   \
        pr[0] = (__bf16)__builtin_amdgcn_exp2f(s[c >> 1][qb][(c & 1) * 8 + j]);      \
        pr[1] = (__bf16)__builtin_amdgcn_exp2f(s[c >> 1][qb][(c & 1) * 8 + j + 1]);  \
        pb[c][qb][j] = pr[0];                                                        \
        pb[c][qb][j + 1] = pr[1];                                                    \
        if (SUM_) ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls, false);         \
      }                                                                              \
    }                                                                                \
    (TS_)[qb] = ls;                                                                  \
  }

  // Softmax of one tile and O^T += V^T P^T with V^T stage SV_.  Lazy max:
  // weights are taken relative to the running max as it stands.  On the
  // first tile the max is set (to 0 when the tile's max is within kHome of
  // it); later, with CHK_, a partial row sum above 2^64 (which any single
  // weight above 2^64 implies) moves the max up to the tile's, rescales O
  // and l, and recomputes the weights.  No weight ever exceeds 2^64 and no
  // column's largest weight falls below 2^-64.  The branch is wave-uniform
  // and rare.  Without CHK_ the row sums go to lsum by MFMA, and such a tile
  // only leaves a sum above 2^64 there (its weights, and all later results,
  // are then discarded).
#define FD_ATT_PV(SV_, TILE_, CHK_)                                                  \
  {                                                                                  \
    const int tile_ = (TILE_);                                                       \
    bf16x8 pb[4][2];                                                                 \
    float ts[2];                                                                     \
    FD_ATT_EXP(ts, CHK_)                                                             \
    const bool need_ = tile_ == 0 || ((CHK_) && (ts[0] > kLazySum || ts[1] > kLazySum)); \
    if (__builtin_amdgcn_ballot_w64(need_)) {                                        \
      _Pragma("unroll") for (int qb = 0; qb < 2; ++qb) {                             \
        float m_ = fmaxf(s[0][qb][0], s[0][qb][1]);                                  \
        _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                             \
        _Pragma("unroll") for (int v = (kb == 0 ? 2 : 0); v < 16; ++v)               \
          m_ = fmaxf(m_, s[kb][qb][v]);                                              \
        const float mall = fmaxf(m_, __shfl_xor(m_, 32));                            \
        const float mnew = tile_ == 0 ? (fabsf(mall) <= kHome ? 0.0f : (float)to_bf16(mall)) \
                                      : (float)to_bf16(mrun[qb] + fmaxf(mall, 0.0f)); \
        const float delta = mnew - mrun[qb];                                         \
        mrun[qb] = mnew;                                                             \
        /* first tile: l and O are still 0, nothing to rescale */                   \
        const float sc = tile_ == 0 ? 1.0f : __builtin_amdgcn_exp2f(-delta);         \
        lrun[qb] *= sc;                                                              \
        _Pragma("unroll") for (int db = 0; db < 2; ++db)                             \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) o[db][qb][v] *= sc;           \
        _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                             \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) s[kb][qb][v] -= delta;        \
        if (half == 0) mext[qb][0] = to_bf16(-mnew);                                 \
      }                                                                              \
      ext_on = __builtin_amdgcn_ballot_w64(mrun[0] != 0.0f || mrun[1] != 0.0f) != 0; \
      FD_ATT_EXP(ts, CHK_)                                                           \
    }                                                                                \
    if (CHK_) {                                                                      \
      lrun[0] += ts[0];                                                              \
      lrun[1] += ts[1];                                                              \
    }                                                                                \
    /* query block 0's MFMAs first: they need only its half of the weights, */  \
    /* so they can run while block 1's weights are still being computed     */  \
    /* (the V fragments are read once per query block)                      */  \
    _Pragma("unroll") for (int qb = 0; qb < 2; ++qb)                                 \
    _Pragma("unroll") for (int c = 0; c < 4; ++c) {                                  \
      const int chunk = (c >> 1) * 4 + (c & 1) * 2 + half;                           \
      bf16x8 vf[2];                                                                  \
      _Pragma("unroll") for (int db = 0; db < 2; ++db) vf[db] =                      \
          *reinterpret_cast<const bf16x8*>((SV_) + swz(db * 32 + r32, chunk));       \
      _Pragma("unroll") for (int db = 0; db < 2; ++db)                               \
        o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pb[c][qb],       \
                                                            o[db][qb], 0, 0, 0);     \
      if (!(CHK_))                                                                   \
        lsum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel16, pb[c][qb],         \
                                                           lsum[qb], 0, 0, 0);       \
    }                                                                                \
  }

  // Ring of STAGES stages; the fetch of tile t + STAGES - 1 is issued right
  // after the barrier of tile t, into the stage tile t - 1 held (every wave
  // is past tile t - 1 there).  Each wave waits at barrier t for its part of
  // tile t.
  constexpr int kWait = (STAGES - 2) * LPW;
#define FD_ATT_STEP(CK_, CV_, NK_, NV_, T_, CHK_, IDLE_)                             \
  {                                                                                  \
    wait_vmcnt<kWait>();                                                             \
    stage_barrier();                                                                 \
    FD_ATT_ISSUE(NK_, NV_)                                                           \
    if (!(IDLE_)) {                                                                  \
      floatx16 s[2][2];                                                              \
      FD_ATT_QK(CK_, t0 + (T_))                                                      \
      FD_ATT_PV(CV_, T_, CHK_)                                                       \
    }                                                                                \
  }
  // All of this split's key tiles.  The whole workgroup shares one split, so
  // the branches on ntiles and tile are uniform.  With IDLE_ the wave only
  // fetches its share of every tile and meets every barrier.
#define FD_ATT_RUN(CHK_, IDLE_)                                                      \
  if (ntiles > 0) {                                                                  \
    FD_ATT_ISSUE(sk0, sv0)                                                           \
    FD_ATT_ISSUE(sk1, sv1)                                                           \
    if constexpr (STAGES == 4) FD_ATT_ISSUE(sk2, sv2)                                \
    if constexpr (STAGES == 3) {                                                     \
      for (int tile = 0; tile < ntiles; tile += 3) {                                 \
        FD_ATT_STEP(sk0, sv0, sk2, sv2, tile, CHK_, IDLE_)                           \
        if (tile + 1 < ntiles) FD_ATT_STEP(sk1, sv1, sk0, sv0, tile + 1, CHK_, IDLE_) \
        if (tile + 2 < ntiles) FD_ATT_STEP(sk2, sv2, sk1, sv1, tile + 2, CHK_, IDLE_) \
      }                                                                              \
    } else {                                                                         \
      for (int tile = 0; tile < ntiles; tile += 4) {                                 \
        FD_ATT_STEP(sk0, sv0, sk3, sv3, tile, CHK_, IDLE_)                           \
        if (tile + 1 < ntiles) FD_ATT_STEP(sk1, sv1, sk0, sv0, tile + 1, CHK_, IDLE_) \
        if (tile + 2 < ntiles) FD_ATT_STEP(sk2, sv2, sk1, sv1, tile + 2, CHK_, IDLE_) \
        if (tile + 3 < ntiles) FD_ATT_STEP(sk3, sv3, sk2, sv2, tile + 3, CHK_, IDLE_) \
      }                                                                              \
    }                                                                                \
    wait_vmcnt<0>();                                                                 \
  }
  // Waves whose 64 queries all lie past n (in a ragged last query tile) only
  // move their share of the tiles: no MFMA or softmax work for padding.
  const bool idle = q0 + wave * 64 >= n;
  if (idle) {
    FD_ATT_RUN(false, true)
  } else {
    FD_ATT_RUN(false, false)
  }
  // Every wave is past its last read of the ring.  A weight above 2^64
  // implies a row sum above 2^64 (and a sum above 2^64 may come from many
  // smaller weights, which only costs a needless second run): if some
  // column's sum passed it, start over from the first tile with the check.
  // An infinite weight makes the MFMA sum NaN (0 times infinity in the
  // unselected lanes), so the test is written to catch NaN as well.
  __syncthreads();
  const bool big_ = !(lsum[0][0] <= kLazySum && lsum[0][1] <= kLazySum &&
                      lsum[1][0] <= kLazySum && lsum[1][1] <= kLazySum);
  if (__builtin_amdgcn_ballot_w64(big_) && lane == 0) rerun = 1;
  __syncthreads();
  const bool checked = rerun != 0;
  if (checked) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      mrun[a] = 0.0f;
      lrun[a] = 0.0f;
      mext[a][0] = to_bf16(0.0f);
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[a][b][v] = 0.0f;
    }
    ext_on = false;
    iss_t = t0;
    iss_f = iss_f0;
    iss_key0 = iss_key00;
    iss_sb = iss_sb0;
    if (idle) {
      FD_ATT_RUN(true, true)
    } else {
      FD_ATT_RUN(true, false)
    }
  }
#undef FD_ATT_RUN
#undef FD_ATT_STEP
#undef FD_ATT_QK
#undef FD_ATT_EXP
#undef FD_ATT_PV
#undef FD_ATT_ISSUE

  // Row sum of this lane's query column of q-block qb: from the two
  // half-waves' dot2 sums after a checked run, else from the MFMA sums
  // (lane q % 16, element q / 16).
  auto row_sum = [&](int qb) {
    if (checked) return lrun[qb] + __shfl_xor(lrun[qb], 32);
    const float a = __shfl(lsum[qb][0], r32 & 15), b = __shfl(lsum[qb][1], r32 & 15);
    return r32 < 16 ? a : b;
  };
  // Normalise and store O[q][head*64 + d] (bf16), or with key splits this
  // split's normalised partial (fp16) and its (max, sum, scale).  O^T block
  // layout: column q = lane % 32, row d = 8 * (v / 4) + 4 * (lane / 32) + v % 4.
  if (splits > 1) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l = row_sum(qb);
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      // fp16 ends at 65504: a partial whose largest entry reaches 2^15 is
      // stored divided by a power of two (exact), so that its largest entry
      // lies in [2^14, 2^15), and the divisor goes to the combine.  Below
      // 2^15 the divisor is 1 and nothing changes.
      float amax = 0.0f;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) amax = fmaxf(amax, fabsf(o[db][qb][v]));
      amax = fmaxf(amax, __shfl_xor(amax, 32)) * inv;
      float sc = 1.0f, sinv = inv;
      if (amax >= 32768.0f) {
        const int e = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 14;
        sc = __uint_as_float((uint32_t)(127 + e) << 23);
        sinv = inv * __uint_as_float((uint32_t)(127 - e) << 23);
      }
      const int q = q0 + wave * 64 + qb * 32 + r32;
      if (q < n) {
        uint16_t* prow = args.part_o + ((size_t)split * n + q) * heads * HD + head * HD;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint2 w;
            w.x = f2h2(o[db][qb][4 * g] * sinv, o[db][qb][4 * g + 1] * sinv);
            w.y = f2h2(o[db][qb][4 * g + 2] * sinv, o[db][qb][4 * g + 3] * sinv);
            *reinterpret_cast<uint2*>(prow + db * 32 + 8 * g + 4 * half) = w;
          }
        if (half == 0)
          *reinterpret_cast<float4*>(args.part_ml +
                                     (((size_t)split * heads + head) * n + q) * 4) =
              make_float4(ntiles > 0 ? mrun[qb] : -1e30f, l, sc, 0.0f);
      }
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = row_sum(qb);
    const float inv = 1.0f / l;
    const int q = q0 + wave * 64 + qb * 32 + r32;
    if (q < n) {
      // Stream b = head / oh owns O rows b n .. b n + n - 1 (oh heads per row).
      const int oh = args.o_heads ? args.o_heads : heads;
      const int ob = head / oh;
      uint16_t* orow = args.o + ((size_t)ob * n + q) * oh * HD + (head - ob * oh) * HD;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * half;
          uint2 w;
          w.x = f2bf2(o[db][qb][4 * g + 0] * inv, o[db][qb][4 * g + 1] * inv);
          w.y = f2bf2(o[db][qb][4 * g + 2] * inv, o[db][qb][4 * g + 3] * inv);
          *reinterpret_cast<uint2*>(orow + d) = w;
        }
    }
  }
}

// Merge the key splits of a head_dim-64 attention: per (query, head),
// O = sum_i w_i O_i / sum_i w_i with w_i = l_i 2^(m_i - max_j m_j), where O_i
// is split i's normalised output (stored as fp16 O_i / c_i, c_i a power of
// two, 1 unless O_i reaches 2^15) and (m_i, l_i) its running max (log2
// units) and sum.  One thread per (query, head, 8 dims): 8 threads share a
// (query, head), read 16 contiguous bytes per split and store 16.  O has oh
// heads per row; head h belongs to stream h / oh (rows (h / oh) n ..).
__global__ __launch_bounds__(256)
void attention_combine_kernel(const uint16_t* part_o, const float* part_ml, int splits,
                              int n, int heads, int oh, uint16_t* o) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int d8 = (int)(idx & 7);
  const long r = idx >> 3;
  const int head = (int)(r % heads);
  const long q = r / heads;
  if (q >= n) return;
  const size_t D = (size_t)heads * 64;
  float4 ml[4];
  float mmax = -1e30f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ml[i] = i < splits ? *reinterpret_cast<const float4*>(
                             part_ml + (((size_t)i * heads + head) * n + q) * 4)
                       : make_float4(-1e30f, 0.0f, 1.0f, 0.0f);
    mmax = fmaxf(mmax, ml[i].x);
  }
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  float wsum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < splits) {
      const float w = ml[i].y * __builtin_amdgcn_exp2f(ml[i].x - mmax);
      const float wc = w * ml[i].z;
      const uint4 hv = *reinterpret_cast<const uint4*>(
          part_o + ((size_t)i * n + q) * D + head * 64 + d8 * 8);
      const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += wc * h2f(hw[e] & 0xFFFFu);
        acc[2 * e + 1] += wc * h2f(hw[e] >> 16);
      }
      wsum += w;
    }
  }
  const float inv = 1.0f / wsum;
  uint4 w4;
  w4.x = f2bf2(acc[0] * inv, acc[1] * inv);
  w4.y = f2bf2(acc[2] * inv, acc[3] * inv);
  w4.z = f2bf2(acc[4] * inv, acc[5] * inv);
  w4.w = f2bf2(acc[6] * inv, acc[7] * inv);
  const int ob = head / oh;
  *reinterpret_cast<uint4*>(o + ((size_t)ob * n + q) * oh * 64 + (head - ob * oh) * 64 +
                            d8 * 8) = w4;
}

// head_dim 16 or 32 (small models): one thread per (head, query), fp32
// online softmax over the cached keys in chronological order.  HD is a
// template argument so that the query row and the accumulator stay in
// registers (every loop over d is unrolled); a key row is two or four
// 16-byte loads.
template <int HD>
__global__ __launch_bounds__(64)
void attention_small_kernel(const AttnArgs args_in) {
  static_assert(HD == 16 || HD == 32, "small head dims");
  const AttnArgs args = args_in;
  const int head = blockIdx.y;
  const int q = blockIdx.x * 64 + threadIdx.x;
  if (q >= args.n) return;
  const int n_pad = args.n_pad, heads = args.heads;
  const DeviceState* st = args.state;
  float qv[HD], acc[HD];
  const uint4* qp =
      reinterpret_cast<const uint4*>(args.q + ((size_t)head * args.q_rows + q) * HD);
#pragma unroll
  for (int c = 0; c < HD / 8; ++c) {
    const uint4 w = qp[c];
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[8 * c + 2 * e] = __uint_as_float(u[e] << 16);
      qv[8 * c + 2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int d = 0; d < HD; ++d) acc[d] = 0.0f;
  float m = -1e30f, l = 0.0f;
  const size_t slot_stride = (size_t)args.kv_heads * n_pad * HD;
  const int kvh = head * args.kv_heads / heads;
  const int n_valid = st->n_valid;
  for (int f = 0; f < n_valid; ++f) {
    const int slot = st->chrono_slot[f];
    const uint16_t* kb = args.ring_k + slot * slot_stride + (size_t)kvh * n_pad * HD;
    const uint16_t* vb = args.ring_vt + slot * slot_stride + (size_t)kvh * HD * n_pad;
    for (int key = 0; key < args.n; ++key) {
      const uint4* kr = reinterpret_cast<const uint4*>(kb + (size_t)key * HD);
      float sc = 0.0f;
#pragma unroll
      for (int c = 0; c < HD / 8; ++c) {
        const uint4 w = kr[c];
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc = fmaf(qv[8 * c + 2 * e], __uint_as_float(u[e] << 16), sc);
          sc = fmaf(qv[8 * c + 2 * e + 1], __uint_as_float(u[e] & 0xFFFF0000u), sc);
        }
      }
      const float mn = fmaxf(m, sc);
      const float alpha = exp2f(m - mn);
      const float p = exp2f(sc - mn);
      l = l * alpha + p;
      const int col = vt_perm(key);
#pragma unroll
      for (int d = 0; d < HD; ++d)
        acc[d] = acc[d] * alpha + p * bf2f(vb[(size_t)d * n_pad + col]);
      m = mn;
    }
  }
  const int oh = args.o_heads ? args.o_heads : heads;
  const int ob = head / oh;
  uint16_t* orow = args.o + ((size_t)ob * args.n + q) * oh * HD + (head - ob * oh) * HD;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < HD; ++d) orow[d] = f2bf(acc[d] * inv);
}

// Test support: scatter plain [f][kv head][n][hd] K and V into ring slots.
__global__ void pack_ring_kernel(const uint16_t* k, const uint16_t* v, int n_frames,
                                 int first_slot, int heads, int n, int n_pad, int hd,
                                 uint16_t* ring_k, uint16_t* ring_vt) {
  // `heads` here counts KV heads.
  const long total = (long)n_frames * heads * n * hd;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int d = (int)(idx % hd);
  long r = idx / hd;
  const int tok = (int)(r % n);
  r /= n;
  const int head = (int)(r % heads);
  const int f = (int)(r / heads);
  const int slot = (first_slot + f) % n_frames;
  const size_t base = ((size_t)slot * heads + head) * (size_t)n_pad * hd;
  ring_k[base + (size_t)tok * hd + d] = k[idx];
  ring_vt[base + (size_t)d * n_pad + vt_perm(tok)] = v[idx];
}

// Test support for the scratch-only entry point: write the ring state
// (a kernel argument), zero n16 16-byte words, copy [heads][n][hd] queries
// into [heads][q_rows][hd] rows.
__global__ void write_state_kernel(DeviceState* st, const DeviceState v) {
  if (threadIdx.x == 0) *st = v;
}

__global__ __launch_bounds__(256)
void zero16_kernel(uint4* p, long n16) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ __launch_bounds__(256)
void copy_q_kernel(const uint16_t* q, long total, int n, int hd, int q_rows, uint16_t* qb) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int d = (int)(i % hd);
  const long r = i / hd;
  const int t = (int)(r % n);
  const long head = r / n;
  qb[(head * q_rows + t) * hd + d] = q[i];
}

}  // namespace

int attention_splits(int heads, int n, int head_dim) {
  if (head_dim != 64 || n <= 0) return 1;
  // Workgroups run in rounds of 256 (one per CU); a split of the cached key
  // tiles costs one round per 256 workgroups times its tiles, and merging
  // the splits costs about two tiles.  Take the cheapest of 1..4 splits
  // (the fewest on a tie), costed on two cached frames whatever the window,
  // so that a frame is computed the same way under every window (frame 0
  // under window 2 equals frame 0 under window 1, bit for bit).
  const long wgs = (long)heads * ((n + 511) / 512);
  const long tiles = 2L * ((n + 63) / 64);
  int best = 1;
  long best_cost = 0;
  for (int sp = 1; sp <= 4; ++sp) {
    const long rounds = (wgs * sp + 255) / 256;
    const long cost = rounds * ((tiles + sp - 1) / sp) + (sp > 1 ? 2 : 0);
    if (sp == 1 || cost < best_cost) { best = sp; best_cost = cost; }
  }
  return best;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  if (a.head_dim == 64) {
    if (a.n_pad % AK != 0) return hipErrorInvalidValue;
    // One head x 512 queries per workgroup (8 waves); when that leaves CUs
    // idle the cached key tiles are split over several workgroups.
    const int qtiles = (a.n + 511) / 512;
    if (a.q_rows < qtiles * 512) return hipErrorInvalidValue;
    if (a.splits < 1 || a.splits > 4) return hipErrorInvalidValue;
    if (a.splits > 1 && (!a.part_o || !a.part_ml)) return hipErrorInvalidValue;
    const int blocks = a.heads * qtiles * a.splits;
    hipLaunchKernelGGL((attention_hd64_kernel<8, 4>), dim3(blocks), dim3(512), 0, s, a);
    if (a.splits > 1) {
      const long threads = (long)a.n * a.heads * 8;
      hipLaunchKernelGGL(attention_combine_kernel, dim3((unsigned)((threads + 255) / 256)),
                         dim3(256), 0, s, a.part_o, a.part_ml, a.splits, a.n, a.heads,
                         a.o_heads ? a.o_heads : a.heads, a.o);
    }
  } else {
    if (a.head_dim != 16 && a.head_dim != 32) return hipErrorInvalidValue;
    dim3 grid((a.n + 63) / 64, a.heads);
    if (a.head_dim == 16)
      hipLaunchKernelGGL(attention_small_kernel<16>, grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL(attention_small_kernel<32>, grid, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace fd

extern "C" fd_status fdk_attention(const uint16_t* q, const uint16_t* k,
                                   const uint16_t* v, int n_frames, int first_slot,
                                   int heads, int kv_heads, int n, int hd, int splits_req,
                                   uint16_t* out, void* stream) {
  using namespace fd;
  if (!q || !k || !v || !out || n_frames < 1 || n_frames > FD_MAX_WINDOW ||
      first_slot < 0 || heads < 1 || n < 1 || kv_heads < 1 || heads % kv_heads ||
      splits_req < 0 || splits_req > 4 || (splits_req > 1 && hd != 64))
    return FD_ERR_INVALID_ARG;
  if (hd != 16 && hd != 32 && hd != 64) return FD_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const int n_pad = (n + 63) / 64 * 64;
  const int q_rows = (n + 511) / 512 * 512;
  const size_t ring_elems = (size_t)n_frames * kv_heads * n_pad * hd;
  const int splits = splits_req ? splits_req : attention_splits(heads, n, hd);
  uint16_t *rk = nullptr, *rv = nullptr, *qb = nullptr;
  uint16_t* po = nullptr;
  float* pml = nullptr;
  DeviceState* st = nullptr;
  fd_status res = FD_OK;
  if (hipMalloc(&rk, ring_elems * 2) != hipSuccess ||
      hipMalloc(&rv, ring_elems * 2) != hipSuccess ||
      hipMalloc(&qb, (size_t)heads * q_rows * hd * 2) != hipSuccess ||
      hipMalloc(&st, sizeof(DeviceState)) != hipSuccess ||
      (splits > 1 &&
       (hipMalloc(&po, (size_t)splits * n * heads * hd * 2) != hipSuccess ||
        hipMalloc(&pml, (size_t)splits * heads * n * 4 * 4) != hipSuccess))) {
    res = FD_ERR_OOM;
  }
  DeviceState hs{};
  hs.frames_done = n_frames;
  hs.t = n_frames - 1;
  hs.n_valid = n_frames;
  for (int i = 0; i < FD_MAX_WINDOW; ++i) {
    hs.slot_frame[i] = -1;
    hs.chrono_slot[i] = i < n_frames ? (first_slot + i) % n_frames : 0;
  }
  for (int f = 0; f < n_frames; ++f) hs.slot_frame[(first_slot + f) % n_frames] = f;
  hs.write_slot = (first_slot + n_frames - 1) % n_frames;
  if (res == FD_OK &&
      (hipMemsetAsync(rk, 0, ring_elems * 2, s) != hipSuccess ||
       hipMemsetAsync(rv, 0, ring_elems * 2, s) != hipSuccess ||
       hipMemsetAsync(qb, 0, (size_t)heads * q_rows * hd * 2, s) != hipSuccess ||
       hipMemcpyAsync(st, &hs, sizeof hs, hipMemcpyHostToDevice, s) != hipSuccess ||
       hipMemcpy2DAsync(qb, (size_t)q_rows * hd * 2, q, (size_t)n * hd * 2,
                        (size_t)n * hd * 2, heads, hipMemcpyDeviceToDevice, s) != hipSuccess))
    res = FD_ERR_DEVICE;
  if (res == FD_OK) {
    const long total = (long)n_frames * kv_heads * n * hd;
    hipLaunchKernelGGL(pack_ring_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                       0, s, k, v, n_frames, first_slot, kv_heads, n, n_pad, hd, rk, rv);
    AttnArgs a{qb, rk, rv, st, out, n, n_pad, q_rows, heads, hd, n_frames, 0.0f,
               po, pml, splits, kv_heads, heads};
    if (hipGetLastError() != hipSuccess || launch_attention(a, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      res = FD_ERR_DEVICE;
  } else {
    (void)hipStreamSynchronize(s);
  }
  if (rk) (void)hipFree(rk);
  if (rv) (void)hipFree(rv);
  if (qb) (void)hipFree(qb);
  if (st) (void)hipFree(st);
  if (po) (void)hipFree(po);
  if (pml) (void)hipFree(pml);
  return res;
}

namespace {
// Device address of `scratch` on each device, looked up once per device
// (with that device current) by hipGetSymbolAddress.
std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {};

fd_status noalloc_scratch(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FD_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return FD_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return FD_ERR_DEVICE;
    }
    g_scratch_dev[dev] = p;
  }
  *out = static_cast<uint8_t*>(g_scratch_dev[dev]);
  return FD_OK;
}
}  // namespace

extern "C" fd_status fdk_attention_noalloc(const uint16_t* q, const uint16_t* k,
                                           const uint16_t* v, int n_frames, int first_slot,
                                           int heads, int kv_heads, int n, int hd,
                                           int splits_req, uint16_t* out, void* stream) {
  using namespace fd;
  if (!q || !k || !v || !out || n_frames < 1 || n_frames > FD_MAX_WINDOW ||
      first_slot < 0 || heads < 1 || n < 1 || kv_heads < 1 || heads % kv_heads ||
      splits_req < 0 || splits_req > 4 || (splits_req > 1 && hd != 64))
    return FD_ERR_INVALID_ARG;
  if (hd != 16 && hd != 32 && hd != 64) return FD_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const long n_pad = (n + 63) / 64 * 64;
  const long q_rows = (n + 511) / 512 * 512;
  const int splits = splits_req ? splits_req : attention_splits(heads, n, hd);
  // Carve the scratch: state, K ring, V^T ring, padded Q (these three zeroed
  // together), then the key-split partials.
  auto up = [](long x) { return (x + 255) / 256 * 256; };
  const long ring_b = (long)n_frames * kv_heads * n_pad * hd * 2;
  const long q_b = (long)heads * q_rows * hd * 2;
  const long o_rk = 256, o_rv = o_rk + up(ring_b), o_q = o_rv + up(ring_b);
  const long o_po = o_q + up(q_b);
  const long po_b = splits > 1 ? (long)splits * n * heads * hd * 2 : 0;
  const long o_pml = o_po + up(po_b);
  const long pml_b = splits > 1 ? (long)splits * heads * n * 4 * 4 : 0;
  const long need = o_pml + up(pml_b);
  if (need > (long)FDK_NOALLOC_SCRATCH_BYTES) return FD_ERR_UNSUPPORTED;
  uint8_t* base = nullptr;
  const fd_status st_ = noalloc_scratch(&base);
  if (st_ != FD_OK) return st_;
  DeviceState* st = reinterpret_cast<DeviceState*>(base);
  uint16_t* rk = reinterpret_cast<uint16_t*>(base + o_rk);
  uint16_t* rv = reinterpret_cast<uint16_t*>(base + o_rv);
  uint16_t* qb = reinterpret_cast<uint16_t*>(base + o_q);
  uint16_t* po = splits > 1 ? reinterpret_cast<uint16_t*>(base + o_po) : nullptr;
  float* pml = splits > 1 ? reinterpret_cast<float*>(base + o_pml) : nullptr;

  DeviceState hs{};
  hs.frames_done = n_frames;
  hs.t = n_frames - 1;
  hs.n_valid = n_frames;
  for (int i = 0; i < FD_MAX_WINDOW; ++i) {
    hs.slot_frame[i] = -1;
    hs.chrono_slot[i] = i < n_frames ? (first_slot + i) % n_frames : 0;
  }
  for (int f = 0; f < n_frames; ++f) hs.slot_frame[(first_slot + f) % n_frames] = f;
  hs.write_slot = (first_slot + n_frames - 1) % n_frames;

  // The previous call's contents are still there: clear ring padding and
  // query padding rows (read by the kernel, never written here) with a fill
  // kernel, then write the state, the ring and the queries.
  const long n16 = (o_po - o_rk) / 16;
  const long kv_total = (long)n_frames * kv_heads * n * hd;
  const long q_total = (long)heads * n * hd;
  hipLaunchKernelGGL(write_state_kernel, dim3(1), dim3(64), 0, s, st, hs);
  hipLaunchKernelGGL(zero16_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(base + o_rk), n16);
  hipLaunchKernelGGL(pack_ring_kernel, dim3((unsigned)((kv_total + 255) / 256)), dim3(256), 0,
                     s, k, v, n_frames, first_slot, kv_heads, n, (int)n_pad, hd, rk, rv);
  hipLaunchKernelGGL(copy_q_kernel, dim3((unsigned)((q_total + 255) / 256)), dim3(256), 0, s,
                     q, q_total, n, hd, (int)q_rows, qb);
  if (hipGetLastError() != hipSuccess) return FD_ERR_DEVICE;
  AttnArgs a{qb, rk, rv, st, out, n, (int)n_pad, (int)q_rows, heads, hd, n_frames, 0.0f,
             po, pml, splits, kv_heads, heads};
  return launch_attention(a, s) == hipSuccess ? FD_OK : FD_ERR_DEVICE;
}
