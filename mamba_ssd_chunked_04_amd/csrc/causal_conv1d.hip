// Depthwise causal conv1d with bias and SiLU for MI355X (gfx950): the step
// before the SSD, page "ops-transformer MambaV2 算子套件", §1.4 (a width-4
// depthwise causal convolution over time, then SiLU) and §4.1
// (mamba2_causal_conv1d: x [B,D,S], per-channel weight and bias):
//
//   out[b,d,t] = act(bias[d] + sum_{k<W} w[d,k] * xx[b,d,t-(W-1)+k])
//
// where xx is x preceded by the W-1 steps of the conv state x_prev (zeros
// without one).  The final conv state is the last W-1 steps of xx.
//
// Pure streaming work (8 bytes of HBM traffic per element), so the kernel is
// shaped around the memory system: one wave64 per (channel row, block of
// 1024 steps), 16-byte loads of four consecutive steps per lane, the three
// steps before a lane's four taken from the lane before it with a DPP wave
// rotation (lane 0 takes them from the previous iteration's lane 63, or, at
// the block start, from memory), non-temporal loads and stores.  Rows whose
// length or addresses do not allow 16-byte access take a one-step-per-lane
// path.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "../../include/ssd_mi355x.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr uint32_t kOOB = 0x80000000u;  // a byte offset past every range: loads 0, stores dropped
constexpr int kStream = 2;              // cache-policy bit nt: data touched once
constexpr int kVec = 4;                 // float4 slots per lane per block
constexpr int kBlockSteps = 64 * 4 * kVec;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ float load1(rsrc_t r, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.f + __expf(-v));
}

// Lane i receives v of lane i-1 (lane 0 receives lane 63): DPP wave_ror:1.
__device__ __forceinline__ float wave_ror1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x13C, 0xf, 0xf, false));
}

struct ConvArgs {
  const float *x, *w, *bias, *x_prev;
  float *out, *fin;
  int64_t rows, dim, S;
  int act;
  uint32_t nblk;  // blocks of kBlockSteps steps per row
};

// Workgroup id -> (first row, step block).  The blocks of one row are
// consecutive ids, so the chip streams each row in address order (measured
// 7-14% faster on rows of 8-16 blocks than taking every row's first block
// first).
__device__ __forceinline__ void decode_block(const ConvArgs &a, int64_t &row0, uint32_t &blk) {
  const uint32_t rg = blockIdx.x / a.nblk;
  blk = blockIdx.x - rg * a.nblk;
  row0 = (int64_t)rg * 4;
}

// Per-row setup shared by both paths: the taps, the bias, the row's buffer
// resources and the step xx(t) for t in [-(W-1), S) read through them.
template <int W>
struct Row {
  rsrc_t rx, rp, ro;
  float tap[W], b;
  __device__ __forceinline__ Row(const ConvArgs &a, int64_t row) {
    const int64_t d = row % a.dim;
    rx = make_rsrc(a.x + row * a.S, (uint32_t)(a.S * 4));
    ro = make_rsrc(a.out + row * a.S, (uint32_t)(a.S * 4));
    rp = make_rsrc(a.x_prev ? a.x_prev + row * (W - 1) : nullptr, a.x_prev ? (W - 1) * 4u : 0u);
#pragma unroll
    for (int k = 0; k < W; ++k) tap[k] = a.w[d * W + k];
    b = a.bias ? a.bias[d] : 0.f;
  }
  // xx(t): x[t] for t >= 0, x_prev[t + W - 1] before (zero without a state);
  // both loads are issued, the one out of its range reads zero
  __device__ __forceinline__ float xx(int64_t t) const {
    const uint32_t ox = t >= 0 ? (uint32_t)t * 4u : kOOB;
    const uint32_t op = t < 0 ? (uint32_t)(t + W - 1) * 4u : kOOB;
    return load1(rx, ox) + load1(rp, op);
  }
};

// The final conv state xx(S-W+1 .. S-1), by lanes 0 .. W-2 of the wave that
// owns a row's last block.
template <int W>
__device__ __forceinline__ void write_final(const ConvArgs &a, const Row<W> &r, int64_t row,
                                            int lane) {
  if (!a.fin || lane >= W - 1) return;
  a.fin[row * (W - 1) + lane] = r.xx(a.S - (W - 1) + lane);
}

// One output from the 7-step window v[0..6] = xx(t-3 .. t+3), t the lane's
// first step, for its step t + e.
template <int W>
__device__ __forceinline__ float tap_sum(const Row<W> &r, const float (&v)[7], int e) {
  float acc = r.b;
#pragma unroll
  for (int k = 0; k < W; ++k) acc = fmaf(r.tap[k], v[4 - W + e + k], acc);
  return acc;
}

// Vector path: S % 4 == 0 and 16-byte aligned x and out.  Wave w of a
// workgroup takes row row0 + w, steps kBlockSteps * blk .. +kBlockSteps;
// lane l holds steps t = t_blk + 4 (l + 64 k), k < kVec.
template <int W>
__global__ __launch_bounds__(256) void causal_conv1d_vec_kernel(ConvArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t row0;
  uint32_t blk;
  decode_block(a, row0, blk);
  const int64_t row = row0 + wave;
  if (row >= a.rows) return;  // the whole wave
  const Row<W> r(a, row);
  const uint32_t tb = blk * kBlockSteps;

  f32x4 cur[kVec];
#pragma unroll
  for (int k = 0; k < kVec; ++k)
    cur[k] = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(r.rx, (tb + 4u * (lane + 64 * k)) * 4u, 0,
                                                     kStream));
  // the three steps before the block: x[tb-3 .. tb-1], or the conv state at
  // tb = 0 (one of the two loads reads zeros)
  const f32x4 pv = __builtin_bit_cast(
      f32x4, __builtin_amdgcn_raw_buffer_load_b128(r.rx, tb > 0 ? (tb - 4) * 4u : kOOB, 0, 0));
  float c[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int m = W - 4 + j;  // x_prev index of step -(3 - j)
    c[j] = pv[1 + j] + (m >= 0 ? load1(r.rp, tb == 0 ? (uint32_t)m * 4u : kOOB) : 0.f);
  }

#pragma unroll
  for (int k = 0; k < kVec; ++k) {
    float rt[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) rt[j] = wave_ror1(cur[k][1 + j]);
    float v[7];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      v[j] = lane == 0 ? c[j] : rt[j];
      c[j] = rt[j];  // lane 0's window start for the next slot: lane 63 of this one
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[3 + e] = cur[k][e];
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float y = tap_sum<W>(r, v, e);
      o[e] = a.act ? silu(y) : y;
    }
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), r.ro,
                                           (tb + 4u * (lane + 64 * k)) * 4u, 0, kStream);
  }
  if (blk == a.nblk - 1) write_final<W>(a, r, row, lane);
}

// General path: lane l of a wave takes steps t = t_blk + l + 64 k, reading
// its window xx(t-W+1 .. t) element by element (neighbouring lanes share the
// cache lines).
template <int W>
__global__ __launch_bounds__(256) void causal_conv1d_step_kernel(ConvArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t row0;
  uint32_t blk;
  decode_block(a, row0, blk);
  const int64_t row = row0 + wave;
  if (row >= a.rows) return;
  const Row<W> r(a, row);
  const int64_t tb = (int64_t)blk * kBlockSteps;
  constexpr int kSteps = kBlockSteps / 64;
  float v[kSteps][W];
#pragma unroll
  for (int k = 0; k < kSteps; ++k)
#pragma unroll
    for (int j = 0; j < W; ++j) v[k][j] = r.xx(tb + lane + 64 * k - (W - 1) + j);
#pragma unroll
  for (int k = 0; k < kSteps; ++k) {
    float acc = r.b;
#pragma unroll
    for (int j = 0; j < W; ++j) acc = fmaf(r.tap[j], v[k][j], acc);
    const int64_t t = tb + lane + 64 * k;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a.act ? silu(acc) : acc), r.ro,
                                          t < a.S ? (uint32_t)t * 4u : kOOB, 0, kStream);
  }
  if (blk == a.nblk - 1) write_final<W>(a, r, row, lane);
}

// ------------------------------------------------------------ token-major layout
// The same convolution on token-major tensors: x [B, S, *] whose token rows
// are xs elements apart (channels 0..D-1 of each row are read, so x may be a
// column range of a wider projection output), out [B, S, D] dense, the conv
// state x_prev / final_state [B, D, W-1] as above.  A wave owns 256 channels
// (4 consecutive ones per lane) and walks TS consecutive steps: every load
// and store of a step is one 1 KB row segment, the W-1 steps before the
// current one stay in registers, and the W-1 steps before the wave's first
// step come from x (or x_prev before t = 0).  Sixteen steps are loaded
// ahead.  Consecutive workgroups take consecutive 256-channel blocks of the
// same steps, so the chip reads and writes whole token rows in address order
// (5-13% faster on the larger shapes than walking one channel block's steps
// first; 16 steps ahead instead of 8 gave another 1-3%).  TS is 32, or 16
// when 32-step waves would give the chip fewer than two workgroups per CU
// (twice the waves for the same bytes: the page's test shape 23.7 -> 22.7
// us; with 512 workgroups already, [4, 2048, 2048] got 9% slower).
constexpr int kTokSteps = 32;   // steps per wave
constexpr int kTokAhead = 16;   // steps loaded ahead

struct TokArgs {
  const float *x, *w, *bias, *x_prev;
  float *out, *fin;
  int64_t batch, dim, S, xs;
  int act;
  uint32_t cblk, sblk;  // 256-channel blocks, 4*TS-step blocks (four waves each)
};

template <int W, int TS>
__global__ __launch_bounds__(256) void causal_conv1d_tok_kernel(TokArgs a) {
  const uint32_t n = blockIdx.x;
  const uint32_t cb = n % a.cblk, sb = (n / a.cblk) % a.sblk;
  const int64_t b = n / (a.sblk * a.cblk);
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int64_t c = 256 * (int64_t)cb + 4 * lane;         // this lane's first channel
  const bool live = c < a.dim;                             // D % 4 == 0: all four or none
  const int64_t t0 = (int64_t)sb * 4 * TS + wave * TS;
  if (t0 >= a.S) return;
  const rsrc_t rx = make_rsrc(a.x + b * a.S * a.xs, (uint32_t)(a.S * a.xs * 4));
  const rsrc_t ro = make_rsrc(a.out + b * a.S * a.dim, (uint32_t)(a.S * a.dim * 4));
  auto xoff = [&](int64_t t) -> uint32_t {
    return (live && t >= 0 && t < a.S) ? (uint32_t)((t * a.xs + c) * 4) : kOOB;
  };
  // taps and bias of the four channels
  f32x4 tap[W], bias = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < W; ++j) tap[j][i] = live ? a.w[(c + i) * W + j] : 0.f;
    if (a.bias && live) bias[i] = a.bias[c + i];
  }
  // the W-1 steps before t0: from x, or from the conv state before t = 0
  f32x4 win[W];  // win[W-1] is filled with the current step
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int64_t t = t0 - (W - 1) + j;
    if (t >= 0) {
      win[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff(t), 0, 0));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        win[j][i] = (a.x_prev && live) ? a.x_prev[((b * a.dim) + c + i) * (W - 1) + (t + W - 1)] : 0.f;
    }
  }
  f32x4 buf[kTokAhead];
#pragma unroll
  for (int k = 0; k < kTokAhead; ++k)
    buf[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff(t0 + k), 0, kStream));
#pragma unroll
  for (int g = 0; g < TS / kTokAhead; ++g) {
#pragma unroll
    for (int k = 0; k < kTokAhead; ++k) {
      const int64_t t = t0 + g * kTokAhead + k;
      win[W - 1] = buf[k];
      if (g + 1 < TS / kTokAhead)
        buf[k] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff(t + kTokAhead), 0, kStream));
      // bias, then the taps oldest first (the channel-major kernels' order)
      f32x4 acc = bias;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < W; ++j) acc[i] = fmaf(tap[j][i], win[j][i], acc[i]);
        if (a.act) acc[i] = silu(acc[i]);
      }
      const uint32_t oo = (live && t < a.S) ? (uint32_t)((t * a.dim + c) * 4) : kOOB;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), ro, oo, 0, kStream);
      // the final conv state: the last W-1 steps of x (x_prev ++ x)
      if (t == a.S - 1 && a.fin && live) {
#pragma unroll
        for (int j = 0; j < W - 1; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) a.fin[((b * a.dim) + c + i) * (W - 1) + j] = win[j + 1][i];
      }
#pragma unroll
      for (int j = 0; j < W - 1; ++j) win[j] = win[j + 1];
    }
  }
}

template <int W>
ssd_status launch_tok(const TokArgs &a, bool short_waves, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.cblk * a.sblk));
  if (short_waves)
    hipLaunchKernelGGL((causal_conv1d_tok_kernel<W, kTokAhead>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((causal_conv1d_tok_kernel<W, kTokSteps>), grid, dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_LAUNCH;
}

template <int W>
ssd_status launch(const ConvArgs &a, bool vec, hipStream_t s) {
  const dim3 grid((unsigned)((a.rows + 3) / 4 * a.nblk));
  if (vec)
    hipLaunchKernelGGL((causal_conv1d_vec_kernel<W>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((causal_conv1d_step_kernel<W>), grid, dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_LAUNCH;
}

bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

bool overlap(const float *a, int64_t na, const float *b, int64_t nb) {
  if (!a || !b) return false;
  return a < b + nb && b < a + na;
}

}  // namespace

extern "C" ssd_status ssd_causal_conv1d(const float *x, const float *w, const float *bias,
                                        const float *x_prev, int64_t batch, int64_t dim,
                                        int64_t seqlen, int64_t width, int activation, float *out,
                                        float *final_state, void *stream) {
  if (!x || !w || !out) return SSD_ERR_INVALID_ARG;
  if (batch < 1 || dim < 1 || seqlen < 1 || width < 1) return SSD_ERR_INVALID_ARG;
  if (activation != 0 && activation != 1) return SSD_ERR_INVALID_ARG;
  const float *ptrs[] = {x, w, bias, x_prev, out, final_state};
  for (const float *p : ptrs)
    if (p && !aligned(p, 4)) return SSD_ERR_INVALID_ARG;
  if (width < 2 || width > 4) return SSD_ERR_UNSUPPORTED;
  const int64_t nblk = (seqlen + kBlockSteps - 1) / kBlockSteps;
  if (batch > ((int64_t)1 << 40) / dim || seqlen * 4 >= ((int64_t)1 << 31) ||
      (batch * dim + 3) / 4 * nblk >= ((int64_t)1 << 31))
    return SSD_ERR_UNSUPPORTED;
  const int64_t n = batch * dim * seqlen, ns = batch * dim * (width - 1);
  if (overlap(out, n, x, n)) return SSD_ERR_INVALID_ARG;  // neighbours' inputs would be overwritten
  // the state may be updated in place when one wave walks each whole row
  if (overlap(final_state, ns, x_prev, ns) && !(final_state == x_prev && seqlen <= kBlockSteps))
    return SSD_ERR_INVALID_ARG;
  ConvArgs a;
  a.x = x;
  a.w = w;
  a.bias = bias;
  a.x_prev = x_prev;
  a.out = out;
  a.fin = final_state;
  a.rows = batch * dim;
  a.dim = dim;
  a.S = seqlen;
  a.act = activation;
  a.nblk = (uint32_t)nblk;
  const bool vec = seqlen % 4 == 0 && aligned(x, 16) && aligned(out, 16);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (width == 2) return launch<2>(a, vec, s);
  if (width == 3) return launch<3>(a, vec, s);
  return launch<4>(a, vec, s);
}

extern "C" ssd_status ssd_causal_conv1d_tokmajor(const float *x, int64_t x_stride, const float *w,
                                                 const float *bias, const float *x_prev,
                                                 int64_t batch, int64_t dim, int64_t seqlen,
                                                 int64_t width, int activation, float *out,
                                                 float *final_state, void *stream) {
  if (!x || !w || !out) return SSD_ERR_INVALID_ARG;
  if (batch < 1 || dim < 1 || seqlen < 1 || width < 1 || x_stride < dim) return SSD_ERR_INVALID_ARG;
  if (activation != 0 && activation != 1) return SSD_ERR_INVALID_ARG;
  const float *ptrs[] = {w, bias, x_prev, final_state};
  for (const float *p : ptrs)
    if (p && !aligned(p, 4)) return SSD_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(out, 16)) return SSD_ERR_INVALID_ARG;
  if (width < 2 || width > 4 || dim % 4 != 0 || x_stride % 4 != 0) return SSD_ERR_UNSUPPORTED;
  const int64_t cblk = (dim + 255) / 256, sblk = (seqlen + 4 * kTokSteps - 1) / (4 * kTokSteps);
  if (seqlen * x_stride * 4 >= ((int64_t)1 << 31) || seqlen * dim * 4 >= ((int64_t)1 << 31) ||
      batch * cblk * sblk >= ((int64_t)1 << 31))
    return SSD_ERR_UNSUPPORTED;
  // out must not overlap x (rows of neighbours would be overwritten); the
  // state may be updated in place only when one wave covers every step (the
  // wave that reads x_prev is then the one that writes final_state)
  if (overlap(out, batch * seqlen * dim, x, (batch * seqlen - 1) * x_stride + dim))
    return SSD_ERR_INVALID_ARG;
  const int64_t ns = batch * dim * (width - 1);
  if (overlap(final_state, ns, x_prev, ns) && !(final_state == x_prev && seqlen <= kTokSteps))
    return SSD_ERR_INVALID_ARG;
  if (overlap(final_state, ns, x, (batch * seqlen - 1) * x_stride + dim) ||
      overlap(out, batch * seqlen * dim, final_state, ns))
    return SSD_ERR_INVALID_ARG;
  TokArgs a;
  a.x = x;
  a.w = w;
  a.bias = bias;
  a.x_prev = x_prev;
  a.out = out;
  a.fin = final_state;
  a.batch = batch;
  a.dim = dim;
  a.S = seqlen;
  a.xs = x_stride;
  a.act = activation;
  // 16-step waves when 32-step ones would leave fewer than two workgroups
  // per CU (256 CUs), unless the state is updated in place over more than
  // 16 steps (one wave must then cover every step)
  const bool in_place = final_state && final_state == x_prev;
  const bool short_waves = batch * cblk * sblk < 2 * 256 && !(in_place && seqlen > kTokAhead);
  const int64_t ts = short_waves ? kTokAhead : kTokSteps;
  a.cblk = (uint32_t)cblk;
  a.sblk = (uint32_t)((seqlen + 4 * ts - 1) / (4 * ts));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (width == 2) return launch_tok<2>(a, short_waves, s);
  if (width == 3) return launch_tok<3>(a, short_waves, s);
  return launch_tok<4>(a, short_waves, s);
}
