// Backward pass of the SSD chunked forward for MI355X (gfx950), fp32.
//
// Gradients of L = <dout, out> + <dfinal_state, final_state> for the forward
// of page "ops-transformer MambaV2 算子套件" §1.1/§1.3 (token recurrence and
// its chunked form) with the tensor semantics of page "Mamba-2 SSD for Ascend
// NPU", "Implementation"; that page's "AscendC training" section and
// "Limitations and roadmap" scope a first backward to contiguous
// P = N = chunk = 64 in FP32, which is the scope here, with the optional z
// gate of the forward (out = y silu(z)) and its gradient.
//
// Per chunk, with delta_j the discretised step, Lam the in-chunk inclusive
// prefix of delta*A (natural log units), S the state entering the chunk and
// G the gradient of the state leaving it:
//   y_i   = sum_{j<=i} (C_i.B_j) e^{Lam_i-Lam_j} delta_j x_j + e^{Lam_i} C_i S + D x_i
//   S_out = e^{Lam_end} S + sum_j e^{Lam_end-Lam_j} delta_j x_j (outer) B_j
// so, with W1_ij = (C_i.B_j) e^{Lam_i-Lam_j} delta_j and
// W2_ij = (dy_i.x_j) e^{Lam_i-Lam_j} delta_j (j <= i):
//   dx_j = sum_i W1_ij dy_i + delta_j e^{Lam_end-Lam_j} G B_j + D dy_j
//   dB_j = sum_i W2_ij C_i + delta_j e^{Lam_end-Lam_j} G^T x_j
//   dC_i = sum_j W2_ij B_j + e^{Lam_i} S^T dy_i
//   G_in = e^{Lam_end} G + sum_i e^{Lam_i} dy_i (outer) C_i       (gradient of S)
// and the step and decay gradients through Lam (reverse in-chunk cumsum of
// dLam gives d(delta*A)), then dt through the clamp and softplus.
//
// Kernels: (1) ssd_bwd_states_kernel, one workgroup per (b, h), walks the
// chunks forward and stores the state entering each; (2) ssd_bwd_chunk_kernel,
// one workgroup per (b, h), walks the chunks backward carrying G in LDS, all
// products as fp32 MFMA tiles (16x16x4) over LDS; (3) ssd_bwd_reduce_kernel
// sums the per-head dB/dC over the heads of a group and dA, dD, ddt_bias over
// the batch.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/ssd_mi355x.h"

namespace {

constexpr int kQ = 64, kP = 64, kN = 64;  // chunk, head dim, state dim
constexpr int kLd = 65;                   // LDS row stride of the 64x64 tiles
constexpr uint32_t kOOB = 0x80000000u;    // a byte offset past every range

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ float ld(rsrc_t r, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

__device__ __forceinline__ void st(rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, 0);
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then row
// totals broadcast to the later rows).
__device__ __forceinline__ float wave_scan(float v) {
  int x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true));
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true));
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true));
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true));
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
  return v;
}

__device__ __forceinline__ float lane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

struct BwdParams {
  const float *x, *dt, *A, *B, *C, *D, *z, *dt_bias, *h0, *dout, *dfin;
  float *dx, *ddt, *dA, *dB, *dC, *dD, *dz, *ddt_bias, *dh0;
  float *states;        // [B*H][nc][P][N]: state entering each chunk
  float *dBh, *dCh;     // [B][L][H][N]: per-head dB, dC
  float *part;          // [B*H][4]: per-(b,h) dA, dD, ddt_bias partial sums
  int64_t batch, L, H, G, nc;
  float dt_min, dt_max;
  int dt_softplus;
};

// silu(v) = v sigmoid(v) and its derivative sigmoid(v) (1 + v (1 - sigmoid(v))).
__device__ __forceinline__ float sigm(float v) { return 1.f / (1.f + __expf(-v)); }

// Per-chunk scalars in LDS.
struct ChunkScalars {
  float lam[kQ], del[kQ], el[kQ], er[kQ], gfac[kQ];  // Lam, delta, e^Lam, e^{Lam_end-Lam}, ddt/ddelta
  float lend, elend;
};

// Raw dt of token t0 + lane (wave 0; zero past the sequence end).
__device__ __forceinline__ float fetch_dt(rsrc_t rdt, uint32_t t0, uint32_t len, uint32_t H,
                                          uint32_t h) {
  const uint32_t j = threadIdx.x & 63;
  return ld(rdt, t0 + j < len ? ((t0 + j) * H + h) * 4u : kOOB);
}

// Discretise the chunk's steps (raw dt of token t0 + j in lane j of wave 0)
// and scan Lam; wave 0 computes, everyone reads after the caller's barrier.
// Tokens past the sequence end get delta = 0.
__device__ __forceinline__ void chunk_scalars(const BwdParams &p, float dt_raw, uint32_t t0,
                                              uint32_t len, float a_h, float bias,
                                              ChunkScalars &cs) {
  if (threadIdx.x >= 64) return;
  const int j = threadIdx.x;
  const bool valid = t0 + j < len;
  const float u = dt_raw + bias;
  float sp = u, dsp = 1.f;
  if (p.dt_softplus) {
    const float e = __expf(-fabsf(u));
    sp = fmaxf(u, 0.f) + log1pf(e);                       // softplus, no overflow
    dsp = u >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);     // sigmoid(u)
  }
  const bool inside = sp >= p.dt_min && sp <= p.dt_max;
  const float delta = valid ? fminf(fmaxf(sp, p.dt_min), p.dt_max) : 0.f;
  const float lam = wave_scan(delta * a_h);
  const float lend = lane63(lam);
  cs.lam[j] = lam;
  cs.del[j] = delta;
  cs.el[j] = __expf(lam);
  cs.er[j] = __expf(lend - lam);
  cs.gfac[j] = (valid && inside) ? dsp : 0.f;
  if (j == 0) {
    cs.lend = lend;
    cs.elend = __expf(lend);
  }
}

// Each thread owns 16 elements of a 64x64 product: rows row_of(r) (four
// consecutive rows of its wave's 16) and columns col_of(c) (one per 16-column
// tile), the accumulator layout of v_mfma_f32_16x16x4f32.
__device__ __forceinline__ int row_of(int r) {
  return 16 * (int)(threadIdx.x >> 6) + 4 * (int)((threadIdx.x & 63) >> 4) + r;
}
__device__ __forceinline__ int col_of(int c) { return 16 * c + (int)(threadIdx.x & 15); }

// acc[r][c] += sum_{k<64} A(row_of(r), k) * B(k, col_of(c)), both in LDS:
// A(i, k) = a[i * ars + k * aks], B(k, j) = b[k * bks + j * bcs].  Wave w
// computes rows 16 w .. 16 w + 15 as four 16x16 tiles with fp32 MFMAs (lane
// l supplies A(16 w + l % 16, k0 + l / 16) and B(k0 + l / 16, 16 c + l % 16)).
__device__ __forceinline__ void mm(const float *a, int ars, int aks, const float *b, int bks,
                                   int bcs, float (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
  const int ai = 16 * (int)(threadIdx.x >> 6) + (lane & 15), kk = lane >> 4;
  f32x4 d[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) d[c] = f32x4{acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
#pragma unroll 4
  for (int k0 = 0; k0 < 64; k0 += 4) {
    const float av = a[ai * ars + (k0 + kk) * aks];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float bv = b[(k0 + kk) * bks + (16 * c + (lane & 15)) * bcs];
      d[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, d[c], 0, 0, 0);
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r][c] = d[c][r];
}

__device__ __forceinline__ void zero(float (&acc)[4][4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
}

// A 64x64 tile in flight in registers: thread t holds rows t/16 + 16 k
// (k < 4), columns 4 (t % 16) .. +3, loaded 16 bytes at a time.
struct Tile4 {
  f32x4 v[4];
};

// Rows t0 .. t0+63 of one (b, h) of a [B, L, X, 64] tensor, zeros past the
// sequence end (t0 = len fetches nothing).  The offsets are selects, never
// branches: a load under a branch makes the compiler wait for every load in
// flight where the paths merge.
__device__ __forceinline__ void fetch_tile(rsrc_t r, uint32_t t0, uint32_t len, uint32_t X,
                                           uint32_t slot, Tile4 &o) {
  const uint32_t c4 = 4 * (threadIdx.x & 15);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t j = (threadIdx.x >> 4) + 16 * k;
    const uint32_t off = t0 + j < len ? (((t0 + j) * X + slot) * 64 + c4) * 4u : kOOB;
    o.v[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
}

// Dense 64x64 tile c of a [nc][64][64] array addressed by r (c = nc, past
// the range, reads zeros).
__device__ __forceinline__ void fetch_dense(rsrc_t r, uint32_t c, Tile4 &o) {
  const uint32_t c4 = 4 * (threadIdx.x & 15);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t j = (threadIdx.x >> 4) + 16 * k;
    o.v[k] = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, ((c * 64 + j) * 64 + c4) * 4u, 0, 0));
  }
}

__device__ __forceinline__ void stage_tile(const Tile4 &o, float *dst) {
  const int c4 = 4 * (threadIdx.x & 15);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = (threadIdx.x >> 4) + 16 * k;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[j * kLd + c4 + e] = o.v[k][e];
  }
}

// The main backward kernel runs eight waves (two per SIMD): wave w takes
// the rows of band w%4 and the columns of half w/4 of every 64x64 product,
// so each thread owns 4 rows x 2 columns (the accumulator layout of
// v_mfma_f32_16x16x4f32 over two 16-column tiles).
constexpr int kT8 = 512;
__device__ __forceinline__ int band8() { return (int)(threadIdx.x >> 6) & 3; }
__device__ __forceinline__ int half8() { return (int)(threadIdx.x >> 8); }
__device__ __forceinline__ int row8(int r) {
  return 16 * band8() + 4 * (int)((threadIdx.x & 63) >> 4) + r;
}
__device__ __forceinline__ int col8(int c) {
  return 16 * (2 * half8() + c) + (int)(threadIdx.x & 15);
}

// acc[r][c] += sum_{k<64} A(row8(r), k) * B(k, col8(c)), as mm with the
// eight-wave split.
__device__ __forceinline__ void mm8(const float *a, int ars, int aks, const float *b, int bks,
                                    int bcs, float (&acc)[4][2]) {
  const int lane = threadIdx.x & 63;
  const int ai = 16 * band8() + (lane & 15), kk = lane >> 4, c0 = 2 * half8();
  f32x4 d[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) d[c] = f32x4{acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
#pragma unroll 4
  for (int k0 = 0; k0 < 64; k0 += 4) {
    const float av = a[ai * ars + (k0 + kk) * aks];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float bv = b[(k0 + kk) * bks + (16 * (c0 + c) + (lane & 15)) * bcs];
      d[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, d[c], 0, 0, 0);
    }
  }
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r][c] = d[c][r];
}

__device__ __forceinline__ void zero8(float (&acc)[4][2]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[r][c] = 0.f;
}

// A 64x64 tile in flight over 512 threads: thread t holds rows t/16 + 32 k
// (k < 2), columns 4 (t % 16) .. +3.
struct Tile2 {
  f32x4 v[2];
};

__device__ __forceinline__ void fetch_tile2(rsrc_t r, uint32_t t0, uint32_t len, uint32_t X,
                                            uint32_t slot, Tile2 &o) {
  const uint32_t c4 = 4 * (threadIdx.x & 15);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t j = (threadIdx.x >> 4) + 32 * k;
    const uint32_t off = t0 + j < len ? (((t0 + j) * X + slot) * 64 + c4) * 4u : kOOB;
    o.v[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
}

__device__ __forceinline__ void fetch_dense2(rsrc_t r, uint32_t c, Tile2 &o) {
  const uint32_t c4 = 4 * (threadIdx.x & 15);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t j = (threadIdx.x >> 4) + 32 * k;
    o.v[k] = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, ((c * 64 + j) * 64 + c4) * 4u, 0, 0));
  }
}

__device__ __forceinline__ void stage_tile2(const Tile2 &o, float *dst) {
  const int c4 = 4 * (threadIdx.x & 15);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int j = (threadIdx.x >> 4) + 32 * k;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[j * kLd + c4 + e] = o.v[k][e];
  }
}

// Workgroup id -> (b, h) pair.  Workgroup n runs on XCD n % 8; the pairs are
// dealt to the XCDs in contiguous runs (the grid is 8 * ceil(B*H / 8)), so
// the heads that share one B/C group run side by side on one XCD and read
// their B and C rows through its L2 instead of each from HBM.  Returns -1
// for the padding workgroups past B*H.
__device__ __forceinline__ int64_t bwd_pair(int64_t total) {
  const int64_t n = blockIdx.x, per = (total + 7) / 8;
  const int64_t t = (n % 8) * per + n / 8;
  return t < total ? t : -1;
}

// Forward pass that stores the state entering every chunk.
__global__ __launch_bounds__(256) void ssd_bwd_states_kernel(BwdParams p) {
  __shared__ float sX[kQ * kLd], sB[kQ * kLd];
  __shared__ ChunkScalars cs;
  const int64_t bh = bwd_pair(p.batch * p.H);
  if (bh < 0) return;
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t g = h / (p.H / p.G);
  const uint32_t H = (uint32_t)p.H, G = (uint32_t)p.G, L = (uint32_t)p.L;
  const rsrc_t rx = make_rsrc(p.x + b * p.L * p.H * kP, L * H * kP * 4u);
  const rsrc_t rb = make_rsrc(p.B + b * p.L * p.G * kN, L * G * kN * 4u);
  const rsrc_t rdt = make_rsrc(p.dt + b * p.L * p.H, L * H * 4u);
  const float a_h = p.A[h], bias = p.dt_bias ? p.dt_bias[h] : 0.f;
  const int tid = threadIdx.x;
  float S[4][4];  // this thread's (p, n) = (row_of(r), col_of(c)) elements of the state
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      S[r][c] = p.h0 ? p.h0[bh * kP * kN + row_of(r) * kN + col_of(c)] : 0.f;
  // the next chunk's x, B and dt are in flight while the current one is used
  Tile4 nx, nb;
  float ndt;
  auto fetch = [&](int64_t cc) {  // cc = nc: nothing (zeros)
    const uint32_t tb = cc < p.nc ? (uint32_t)cc * kQ : L;
    fetch_tile(rx, tb, L, H, (uint32_t)h, nx);
    fetch_tile(rb, tb, L, G, (uint32_t)g, nb);
    ndt = fetch_dt(rdt, tb, L, H, (uint32_t)h);
  };
  fetch(0);
  for (int64_t c = 0; c < p.nc; ++c) {
    const uint32_t t0 = (uint32_t)(c * kQ);
    float *dst = p.states + (bh * p.nc + c) * (kP * kN);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) dst[row_of(r) * kN + col_of(cc)] = S[r][cc];
    __syncthreads();  // the previous chunk's readers of sX/sB/cs are done
    chunk_scalars(p, ndt, t0, L, a_h, bias, cs);
    stage_tile(nx, sX);
    stage_tile(nb, sB);
    fetch(c + 1);
    __syncthreads();
    // weight x_j by e^{Lam_end - Lam_j} delta_j in place (row j)
    for (int e = tid; e < 64 * 64; e += 256) {
      const int j = e >> 6, cc = e & 63;
      sX[j * kLd + cc] *= cs.er[j] * cs.del[j];
    }
    __syncthreads();
    float acc[4][4];
    zero(acc);
    mm(sX, 1, kLd, sB, kLd, 1, acc);  // X^T diag(w) B: A(p, j) = sX[j][p]
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) S[r][cc] = cs.elend * S[r][cc] + acc[r][cc];
  }
}

// Backward: one workgroup per (b, h) walking the chunks from the last.
__global__ __launch_bounds__(kT8) void ssd_bwd_chunk_kernel(BwdParams p) {
  __shared__ float sX[kQ * kLd], sDY[kQ * kLd], sB[kQ * kLd], sC[kQ * kLd];
  __shared__ float sS[kP * kLd], sG[kP * kLd];
  __shared__ float sW1[kQ * kLd], sW2[kQ * kLd];
  // partial sums: per column 16 (the row groups of a half), per row 32 (the
  // column lanes of both halves)
  __shared__ float sPart[kQ * 33], sRowPart[kQ * 33], sColPart[kQ * 17];
  __shared__ float sRed[kT8 / 64];
  __shared__ float sVec[6][kQ];  // q, r, w, v, dLam, (spare)
  __shared__ ChunkScalars cs;

  const int64_t bh = bwd_pair(p.batch * p.H);
  if (bh < 0) return;
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t g = h / (p.H / p.G);
  const uint32_t H = (uint32_t)p.H, G = (uint32_t)p.G, L = (uint32_t)p.L;
  const rsrc_t rx = make_rsrc(p.x + b * p.L * p.H * kP, L * H * kP * 4u);
  const rsrc_t rdy = make_rsrc(p.dout + b * p.L * p.H * kP, L * H * kP * 4u);
  const rsrc_t rb = make_rsrc(p.B + b * p.L * p.G * kN, L * G * kN * 4u);
  const rsrc_t rc = make_rsrc(p.C + b * p.L * p.G * kN, L * G * kN * 4u);
  const rsrc_t rdt = make_rsrc(p.dt + b * p.L * p.H, L * H * 4u);
  const rsrc_t rdx = make_rsrc(p.dx + b * p.L * p.H * kP, L * H * kP * 4u);
  const rsrc_t rdb = make_rsrc(p.dBh + b * p.L * p.H * kN, L * H * kN * 4u);
  const rsrc_t rdc = make_rsrc(p.dCh + b * p.L * p.H * kN, L * H * kN * 4u);
  const rsrc_t rddt = make_rsrc(p.ddt + b * p.L * p.H, L * H * 4u);
  // the gate (optional): dy = dout silu(z), dz = dout silu'(z) y_pre
  const bool gated = p.z != nullptr;
  const rsrc_t rz = make_rsrc(gated ? p.z + b * p.L * p.H * kP : nullptr, gated ? L * H * kP * 4u : 0u);
  const rsrc_t rdz = make_rsrc(gated ? p.dz + b * p.L * p.H * kP : nullptr, gated ? L * H * kP * 4u : 0u);
  const float a_h = p.A[h], bias = p.dt_bias ? p.dt_bias[h] : 0.f;
  const float Dh = p.D ? p.D[h] : 0.f;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // G = dfinal_state (or zero)
  for (int e = tid; e < kP * kN; e += kT8)
    sG[(e >> 6) * kLd + (e & 63)] = p.dfin ? p.dfin[bh * kP * kN + e] : 0.f;
  float accA = 0.f, accD = 0.f, accBias = 0.f;  // wave 0 / all threads' shares

  // the next chunk's tiles are in flight while the current one is computed
  const rsrc_t rs = make_rsrc(p.states + bh * p.nc * (kP * kN), (uint32_t)(p.nc * kP * kN * 4));
  Tile2 nx, ndy, nb, ncc, ns, nz;
  float ndt;
  auto fetch = [&](int64_t cc) {  // cc = -1: nothing (zeros)
    const uint32_t tb = cc >= 0 ? (uint32_t)cc * kQ : L;
    const uint32_t cd = cc >= 0 ? (uint32_t)cc : (uint32_t)p.nc;
    fetch_tile2(rx, tb, L, H, (uint32_t)h, nx);
    fetch_tile2(rdy, tb, L, H, (uint32_t)h, ndy);
    fetch_tile2(rb, tb, L, G, (uint32_t)g, nb);
    fetch_tile2(rc, tb, L, G, (uint32_t)g, ncc);
    fetch_dense2(rs, cd, ns);
    ndt = fetch_dt(rdt, tb, L, H, (uint32_t)h);
    fetch_tile2(rz, tb, L, H, (uint32_t)h, nz);  // zeros without a gate
  };
  fetch(p.nc - 1);

  for (int64_t c = p.nc - 1; c >= 0; --c) {
    const uint32_t t0 = (uint32_t)(c * kQ);
    __syncthreads();  // the previous chunk is done with every LDS array
    chunk_scalars(p, ndt, t0, L, a_h, bias, cs);
    stage_tile2(nx, sX);
    // dy = dout silu(z) into LDS; gz = dout silu'(z) stays in registers for
    // dz, in the same (fetch) element order
    f32x4 gz[2];
    if (gated) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float zz = nz.v[k][e], sg = sigm(zz), dout = ndy.v[k][e];
          ndy.v[k][e] = dout * zz * sg;
          gz[k][e] = dout * sg * (1.f + zz * (1.f - sg));
        }
    }
    stage_tile2(ndy, sDY);
    stage_tile2(nb, sB);
    stage_tile2(ncc, sC);
    stage_tile2(ns, sS);
    fetch(c - 1);  // before the first chunk: zeros, unused
    __syncthreads();

    // dD share: sum of dout * x over the chunk
    for (int e = tid; e < 64 * 64; e += kT8) accD += sDY[(e >> 6) * kLd + (e & 63)] * sX[(e >> 6) * kLd + (e & 63)];

    // CB_ij = C_i.B_j and DX_ij = dy_i.x_j, then the masked weights
    {
      float cb[4][2], dxm[4][2];
      zero8(cb);
      zero8(dxm);
      mm8(sC, kLd, 1, sB, 1, kLd, cb);    // A(i, n) = C[i][n], B(n, j) = B[j][n]
      mm8(sDY, kLd, 1, sX, 1, kLd, dxm);  // A(i, p) = dy[i][p], B(p, j) = x[j][p]
      // T_ij = (C_i.B_j) e^{Lam_i-Lam_j} (dy_i.x_j): its column sums
      // q_j = sum_{i>=j} T_ij (the direct intra gradient of delta_j) and row
      // sums r_i = sum_{j<=i} T_ij delta_j (the intra part of dLam_i), summed
      // per 4x4 tile here and across tiles below
      float colp[2] = {0.f, 0.f}, rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int i = row8(r), j = col8(cc);
          // e^{Lam_i-Lam_j} for j <= i, e^{-inf} = 0 above the diagonal (a
          // select, not a branch per element)
          const float lij = __expf(j <= i ? cs.lam[i] - cs.lam[j] : -INFINITY);
          const float cbl = cb[r][cc] * lij;
          const float t = cbl * dxm[r][cc];
          const float w1 = cbl * cs.del[j];
          const float w2 = dxm[r][cc] * lij * cs.del[j];
          sW1[i * kLd + j] = w1;
          sW2[i * kLd + j] = w2;
          colp[cc] += t;
          rowp[r] += t * cs.del[j];
        }
      const int rgrp = 4 * band8() + (lane >> 4), clane = (tid & 15) + 16 * half8();
#pragma unroll
      for (int k = 0; k < 2; ++k) sColPart[col8(k) * 17 + rgrp] = colp[k];   // 16 row groups
#pragma unroll
      for (int k = 0; k < 4; ++k) sRowPart[row8(k) * 33 + clane] = rowp[k];  // 32 column lanes
    }
    __syncthreads();
    if (tid < 64) {
      float q = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) q += sColPart[tid * 17 + k];
      sVec[0][tid] = q;
    } else if (tid < 128) {
      const int i = tid - 64;
      float r = 0.f;
#pragma unroll
      for (int k = 0; k < 32; ++k) r += sRowPart[i * 33 + k];
      sVec[1][i] = r;
    }

    // dx_j = sum_i W1_ij dy_i + delta_j e^{Lam_end-Lam_j} (B G^T)_j + D dy_j
    {
      float a1[4][2], a2[4][2];
      zero8(a1);
      zero8(a2);
      mm8(sW1, 1, kLd, sDY, kLd, 1, a1);  // A(j, i) = W1[i][j], B(i, p) = dy[i][p]
      mm8(sB, kLd, 1, sG, 1, kLd, a2);    // A(j, n) = B[j][n], B(n, p) = G[p][n]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = row8(r);
        const float f = cs.del[j] * cs.er[j];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int pp = col8(cc);
          const float v = a1[r][cc] + f * a2[r][cc] + Dh * sDY[j * kLd + pp];
          st(rdx, t0 + j < L ? (((t0 + j) * H + (uint32_t)h) * kP + pp) * 4u : kOOB, v);
        }
      }
    }
    // the gate gradient: y_pre = W1 x + e^{Lam} C S^T + D x, recomputed, and
    // dz = dout silu'(z) y_pre; y_pre goes through sW1 (no longer read) to
    // the fetch element order of gz
    if (gated) {
      float a8[4][2];
      zero8(a8);
      mm8(sW1, kLd, 1, sX, kLd, 1, a8);   // A(i, j) = W1[i][j], B(j, p) = x[j][p]
      float a9[4][2];
      zero8(a9);
      mm8(sC, kLd, 1, sS, 1, kLd, a9);    // A(i, n) = C[i][n], B(n, p) = S[p][n]
      __syncthreads();                    // every wave is done reading sW1
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = row8(r);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int pp = col8(cc);
          sW1[i * kLd + pp] = a8[r][cc] + cs.el[i] * a9[r][cc] + Dh * sX[i * kLd + pp];
        }
      }
      __syncthreads();
      const uint32_t c4 = 4 * (tid & 15);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t j = (tid >> 4) + 32 * k;
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = gz[k][e] * sW1[j * kLd + c4 + e];
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, o), rdz,
            t0 + j < L ? (((t0 + j) * H + (uint32_t)h) * kP + c4) * 4u : kOOB, 0, 0);
      }
    }
    // dB_j = sum_i W2_ij C_i + delta_j e^{Lam_end-Lam_j} (X G)_j; w_j = (X G)_j . B_j
    {
      float a3[4][2], a4[4][2];
      zero8(a3);
      zero8(a4);
      mm8(sW2, 1, kLd, sC, kLd, 1, a3);   // A(j, i) = W2[i][j], B(i, n) = C[i][n]
      mm8(sX, kLd, 1, sG, kLd, 1, a4);    // A(j, p) = x[j][p], B(p, n) = G[p][n]
      float wpart[4];
      const int clane = (tid & 15) + 16 * half8();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = row8(r);
        const float f = cs.del[j] * cs.er[j];
        wpart[r] = 0.f;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int n = col8(cc);
          st(rdb, t0 + j < L ? (((t0 + j) * H + (uint32_t)h) * kN + n) * 4u : kOOB,
             a3[r][cc] + f * a4[r][cc]);
          wpart[r] += a4[r][cc] * sB[j * kLd + n];
        }
        sPart[j * 33 + clane] = wpart[r];
      }
    }
    __syncthreads();
    if (tid < 64) {
      float s = 0.f;
      for (int k = 0; k < 32; ++k) s += sPart[tid * 33 + k];
      sVec[2][tid] = s;  // w_j
    }
    __syncthreads();
    // dC_i = sum_j W2_ij B_j + e^{Lam_i} (dy S)_i; v_i = (dy S)_i . C_i
    {
      float a5[4][2], a6[4][2];
      zero8(a5);
      zero8(a6);
      mm8(sW2, kLd, 1, sB, kLd, 1, a5);   // A(i, j) = W2[i][j], B(j, n) = B[j][n]
      mm8(sDY, kLd, 1, sS, kLd, 1, a6);   // A(i, p) = dy[i][p], B(p, n) = S[p][n]
      const int clane = (tid & 15) + 16 * half8();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = row8(r);
        float vpart = 0.f;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int n = col8(cc);
          st(rdc, t0 + i < L ? (((t0 + i) * H + (uint32_t)h) * kN + n) * 4u : kOOB,
             a5[r][cc] + cs.el[i] * a6[r][cc]);
          vpart += a6[r][cc] * sC[i * kLd + n];
        }
        sPart[i * 33 + clane] = vpart;
      }
    }
    // <G, S> shares
    {
      float gs = 0.f;
      for (int e = tid; e < kP * kN; e += kT8) gs += sG[(e >> 6) * kLd + (e & 63)] * sS[(e >> 6) * kLd + (e & 63)];
      gs = lane63(wave_scan(gs));
      if (lane == 0) sRed[wv] = gs;
    }
    __syncthreads();
    if (tid < 64) {
      float s = 0.f;
      for (int k = 0; k < 32; ++k) s += sPart[tid * 33 + k];
      sVec[3][tid] = s;  // v_i
    }
    __syncthreads();

    // token scalars (wave 0): dLam, the reverse cumsum, d delta, ddt, dA
    if (tid < 64) {
      const int k = tid;
      const float dl = cs.del[k], er = cs.er[k];
      const float w = sVec[2][k], U = dl * er * w;
      float dlam = sVec[1][k] - dl * sVec[0][k] + cs.el[k] * sVec[3][k] - U;
      float gsum = 0.f;
#pragma unroll
      for (int q = 0; q < kT8 / 64; ++q) gsum += sRed[q];
      const float usum = lane63(wave_scan(U));
      if (k == 63) dlam += cs.elend * gsum + usum;  // Lam_end = Lam_63
      const float incl = wave_scan(dlam);
      const float da = lane63(incl) - (incl - dlam);  // sum_{m>=k} dLam_m
      const float ddelta = sVec[0][k] + er * w + a_h * da;
      const float ddt = ddelta * cs.gfac[k];
      st(rddt, t0 + k < L ? ((t0 + k) * H + (uint32_t)h) * 4u : kOOB, ddt);
      accA += lane63(wave_scan(dl * da));
      accBias += lane63(wave_scan(ddt));
    }
    __syncthreads();  // every reader of G and S above is done

    // G <- e^{Lam_end} G + sum_i e^{Lam_i} dy_i (outer) C_i
    {
      float a7[4][2];
      zero8(a7);
      // scale dy rows by e^{Lam_i} in place (dy is not read again this chunk)
      for (int e = tid; e < 64 * 64; e += kT8) sDY[(e >> 6) * kLd + (e & 63)] *= cs.el[e >> 6];
      __syncthreads();
      mm8(sDY, 1, kLd, sC, kLd, 1, a7);   // A(p, i) = dy[i][p], B(i, n) = C[i][n]
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          float &gv = sG[row8(r) * kLd + col8(cc)];
          gv = cs.elend * gv + a7[r][cc];
        }
    }
  }
  __syncthreads();
  if (p.dh0)
    for (int e = tid; e < kP * kN; e += kT8) p.dh0[bh * kP * kN + e] = sG[(e >> 6) * kLd + (e & 63)];
  // per-(b, h) partial sums: dA, ddt_bias from wave 0, dD from every thread
  accD = lane63(wave_scan(accD));
  __syncthreads();
  if (lane == 0) sRed[wv] = accD;
  __syncthreads();
  if (tid == 0) {
    p.part[bh * 4 + 0] = accA;
    float sd = 0.f;
#pragma unroll
    for (int q = 0; q < kT8 / 64; ++q) sd += sRed[q];
    p.part[bh * 4 + 1] = sd;
    p.part[bh * 4 + 2] = accBias;
  }
}

// dB, dC: sum of the per-head values over the heads of each group; dA, dD,
// ddt_bias: sums of the per-(b, h) partials over the batch.
__global__ __launch_bounds__(256) void ssd_bwd_reduce_kernel(BwdParams p) {
  const int64_t hpg = p.H / p.G;
  const int64_t n_bc = p.batch * p.L * p.G * kN;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n_bc) {
    const int64_t n = e % kN, rest = e / kN, gg = rest % p.G, bt = rest / p.G;
    float sb = 0.f, sc = 0.f;
    for (int64_t k = 0; k < hpg; ++k) {
      const int64_t src = (bt * p.H + gg * hpg + k) * kN + n;
      sb += p.dBh[src];
      sc += p.dCh[src];
    }
    p.dB[e] = sb;
    p.dC[e] = sc;
  }
  if (e < p.H) {
    float sa = 0.f, sd = 0.f, sbias = 0.f;
    for (int64_t bb = 0; bb < p.batch; ++bb) {
      sa += p.part[(bb * p.H + e) * 4 + 0];
      sd += p.part[(bb * p.H + e) * 4 + 1];
      sbias += p.part[(bb * p.H + e) * 4 + 2];
    }
    p.dA[e] = sa;
    if (p.dD) p.dD[e] = sd;
    if (p.ddt_bias) p.ddt_bias[e] = sbias;
  }
}

size_t align_up(size_t v) { return (v + 255) / 256 * 256; }

struct BwdWs {
  size_t states, dbh, dch, part;
  size_t total() const { return states + dbh + dch + part; }
};

BwdWs bwd_ws(const ssd_desc *d) {
  const int64_t nc = (d->seqlen + kQ - 1) / kQ;
  BwdWs w;
  w.states = align_up((size_t)(d->batch * d->nheads * nc) * kP * kN * 4);
  w.dbh = align_up((size_t)(d->batch * d->seqlen * d->nheads) * kN * 4);
  w.dch = w.dbh;
  w.part = align_up((size_t)(d->batch * d->nheads) * 4 * 4);
  return w;
}

ssd_status check_bwd(const ssd_desc *d, int64_t chunk) {
  if (!d) return SSD_ERR_INVALID_ARG;
  if (d->batch < 1 || d->seqlen < 1 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
      d->ngroups < 1 || chunk < 1 || d->nheads % d->ngroups != 0)
    return SSD_ERR_INVALID_ARG;
  if (!(d->dt_min <= d->dt_max)) return SSD_ERR_INVALID_ARG;
  if (d->bc_dtype != SSD_F32 && d->bc_dtype != SSD_BF16 && d->bc_dtype != SSD_F16)
    return SSD_ERR_INVALID_ARG;
  if (d->headdim != kP || d->dstate != kN || chunk != kQ) return SSD_ERR_UNSUPPORTED;
  if (d->x_dtype != SSD_F32 || d->bc_dtype != SSD_F32 || (d->z && d->z_dtype != SSD_F32) ||
      d->cu_seqlens || d->x_stride || d->bc_stride || d->z_stride || d->dt_stride ||
      d->norm_weight)
    return SSD_ERR_UNSUPPORTED;
  // 32-bit byte offsets within one batch row, 32-bit grid
  if (d->seqlen * d->nheads * kP * 4 >= ((int64_t)1 << 31) || d->batch * d->nheads >= ((int64_t)1 << 31))
    return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

bool aligned4(const void *ptr) { return ((uintptr_t)ptr & 3u) == 0; }

}  // namespace

extern "C" {

ssd_status ssd_bwd_workspace_size(const ssd_desc *d, int64_t chunk, size_t *bytes) {
  if (!bytes) return SSD_ERR_INVALID_ARG;
  const ssd_status s = check_bwd(d, chunk);
  if (s != SSD_OK) return s;
  *bytes = bwd_ws(d).total();
  return SSD_OK;
}

ssd_status ssd_bwd(const float *x, const float *dt, const float *A, const float *B,
                   const float *C, const float *D, int64_t chunk, int dt_softplus,
                   const float *dout, const float *dfinal_state, float *dx, float *ddt,
                   float *dA, float *dB, float *dC, float *dD, float *dz, float *ddt_bias,
                   float *dinitial_state, void *stream, const ssd_desc *d) {
  const ssd_status s = check_bwd(d, chunk);
  if (s != SSD_OK) return s;
  if (!x || !dt || !A || !B || !C || !dout || !dx || !ddt || !dA || !dB || !dC)
    return SSD_ERR_INVALID_ARG;
  if ((D && !dD) || (d->dt_bias && !ddt_bias) || (d->z && !dz)) return SSD_ERR_INVALID_ARG;
  const void *ptrs[] = {x, dt, A, B, C, D, dout, dfinal_state, dx, ddt, dA, dB, dC, dD,
                        dz, ddt_bias, dinitial_state, d->dt_bias, d->initial_state, d->z,
                        d->workspace};
  for (const void *q : ptrs)
    if (q && !aligned4(q)) return SSD_ERR_INVALID_ARG;
  const BwdWs w = bwd_ws(d);
  if (!d->workspace || d->workspace_bytes < w.total()) return SSD_ERR_WORKSPACE;

  BwdParams p;
  memset(&p, 0, sizeof(p));
  p.x = x;
  p.dt = dt;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.dt_bias = d->dt_bias;
  p.h0 = d->initial_state;
  p.dout = dout;
  p.dfin = dfinal_state;
  p.dx = dx;
  p.ddt = ddt;
  p.dA = dA;
  p.dB = dB;
  p.dC = dC;
  p.dD = D ? dD : nullptr;
  p.ddt_bias = d->dt_bias ? ddt_bias : nullptr;
  p.dh0 = dinitial_state;
  p.z = static_cast<const float *>(d->z);
  p.dz = d->z ? dz : nullptr;
  char *ws = static_cast<char *>(d->workspace);
  p.states = reinterpret_cast<float *>(ws);
  p.dBh = reinterpret_cast<float *>(ws + w.states);
  p.dCh = reinterpret_cast<float *>(ws + w.states + w.dbh);
  p.part = reinterpret_cast<float *>(ws + w.states + w.dbh + w.dch);
  p.batch = d->batch;
  p.L = d->seqlen;
  p.H = d->nheads;
  p.G = d->ngroups;
  p.nc = (d->seqlen + kQ - 1) / kQ;
  p.dt_min = d->dt_min;
  p.dt_max = d->dt_max;
  p.dt_softplus = dt_softplus ? 1 : 0;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned nbh = (unsigned)((d->batch * d->nheads + 7) / 8 * 8);  // see bwd_pair
  hipLaunchKernelGGL(ssd_bwd_states_kernel, dim3(nbh), dim3(256), 0, st, p);
  // the descriptor's measurement events bracket the main (chunk) kernel
  if (d->ev_main_begin && hipEventRecord(static_cast<hipEvent_t>(d->ev_main_begin), st) != hipSuccess)
    return SSD_ERR_LAUNCH;
  hipLaunchKernelGGL(ssd_bwd_chunk_kernel, dim3(nbh), dim3(kT8), 0, st, p);
  if (d->ev_main_end && hipEventRecord(static_cast<hipEvent_t>(d->ev_main_end), st) != hipSuccess)
    return SSD_ERR_LAUNCH;
  const int64_t n_bc = d->batch * d->seqlen * d->ngroups * kN;
  const int64_t n_red = n_bc > d->nheads ? n_bc : d->nheads;
  hipLaunchKernelGGL(ssd_bwd_reduce_kernel, dim3((unsigned)((n_red + 255) / 256)), dim3(256), 0,
                     st, p);
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_LAUNCH;
}

}  // extern "C"
