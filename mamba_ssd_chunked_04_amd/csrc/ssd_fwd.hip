// Mamba-2 SSD chunked forward for MI355X (gfx950, CDNA4): HIP kernels and the
// C ABI declared in include/ssd_mi355x.h.
//
// The chunked algorithm follows page "ops-transformer MambaV2 算子套件", §1.3
// (intra-chunk matrix products plus an inter-chunk state recurrence) and the
// operator chain of its §2 / §4.2-§4.5:
//   chunk_cumsum   delta = clamp(softplus(dt + dt_bias)), Lam = in-chunk
//                  inclusive prefix of delta*A, Lam_end = its last value
//   chunk_state    S_loc = sum_i exp(Lam_end - Lam_i) delta_i x_i (outer) B_i
//   state_passing  S_in[c+1] = exp(Lam_end[c]) S_in[c] + S_loc[c]
//   chunk_scan     y_i = sum_{j<=i} (C_i.B_j) exp(Lam_i - Lam_j) delta_j x_j
//                        + exp(Lam_i) C_i . S_in[c]  + D x_i,  then * silu(z_i)
//
// MI355X design (not the Ascend Cube/Vector split of the pages):
//   * one workgroup (4 wave64s) walks `cpg` consecutive chunks of one (b, h),
//     keeping the P x N state in MFMA accumulators across chunks, so the
//     state recurrence costs no HBM traffic inside a chunk group;
//   * when (b, h) pairs alone cannot fill 256 CUs, the sequence is cut into
//     chunk groups: a first pass (ssd_group_state_kernel) builds each
//     group's state from zero, a light elementwise sweep
//     (ssd_group_passing_kernel) chains them, and the main pass
//     (ssd_chunk_scan_kernel) starts every group from its entering state;
//   * all contractions (C.B^T, M.X, C.S^T, X^T.diag(w).B) are
//     v_mfma_f32_16x16x32_f16 tiles (or 16x16x4 fp32 on the check path) with
//     B, X staged in LDS 64 tokens at a time and C held in registers;
//   * the masked C.B^T block is computed transposed, so its accumulator
//     layout is directly the A operand of the M.X product (no LDS round trip);
//   * workgroup ids are swizzled so heads sharing a B/C group run on the same
//     XCD (shared L2).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/ssd_mi355x.h"

namespace {

constexpr int kThreads = 256;   // 4 wave64s
constexpr int kJB = 64;         // tokens per LDS-staged block
constexpr int kP = 64;          // compiled head dim
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- operand types
template <bool F32> struct Mma;
template <> struct Mma<false> {
  using T = _Float16;
  using frag = f16x8;
  using quad = f16x4;
};
template <> struct Mma<true> {
  using T = float;
  using frag = f32x8;
  using quad = f32x4;
};

// D += A.B over one 32-wide K block.  Lane l holds A row (l%16) and B column
// (l%16), eight K values each (the same eight K indices in A and B), and the
// 16x16 result rows 4*(l/16)..+3 of column l%16.
__device__ __forceinline__ f32x4 mma(const f16x8 &a, const f16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8 &a, const f32x8 &b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 8; ++s)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// ---------------------------------------------------------------- storage I/O
struct IoF32 {
  using raw = float;
};
struct IoBF16 {
  using raw = uint16_t;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t v) {
  return __uint_as_float(v << 16);
}

// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <class IO> __device__ __forceinline__ f32x4 load4(const void *base, int64_t idx);
template <> __device__ __forceinline__ f32x4 load4<IoF32>(const void *base, int64_t idx) {
  return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + idx);
}
template <> __device__ __forceinline__ f32x4 load4<IoBF16>(const void *base, int64_t idx) {
  uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + idx);
  f32x4 r;
  r[0] = bf16_bits_to_f32(v.x & 0xffffu);
  r[1] = bf16_bits_to_f32(v.x >> 16);
  r[2] = bf16_bits_to_f32(v.y & 0xffffu);
  r[3] = bf16_bits_to_f32(v.y >> 16);
  return r;
}

template <class IO> __device__ __forceinline__ float load1(const void *base, int64_t idx);
template <> __device__ __forceinline__ float load1<IoF32>(const void *base, int64_t idx) {
  return static_cast<const float *>(base)[idx];
}
template <> __device__ __forceinline__ float load1<IoBF16>(const void *base, int64_t idx) {
  return bf16_bits_to_f32(static_cast<const uint16_t *>(base)[idx]);
}

// Eight consecutive elements converted to the MMA operand type.
template <class IO, bool F32>
__device__ __forceinline__ typename Mma<F32>::frag load8(const void *base, int64_t idx) {
  f32x4 lo = load4<IO>(base, idx), hi = load4<IO>(base, idx + 4);
  typename Mma<F32>::frag r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (typename Mma<F32>::T)lo[e];
    r[4 + e] = (typename Mma<F32>::T)hi[e];
  }
  return r;
}

// ---------------------------------------------------------------- parameters
struct Params {
  const void *x;
  const float *dt;
  const float *A;
  const void *B;
  const void *C;
  const float *D;
  const void *z;
  const float *dt_bias;
  const float *h0;
  void *out;
  float *final_state;
  float *grp_state;  // [B*H][ngroups-1][P*N]: group aggregates, then entering states
  float *grp_lam;    // [B*H][ngroups-1]: group total log2-decay
  int64_t batch, L, H, G, nc, ngroups, cpg;
  float dt_min, dt_max;
  int dt_softplus, z_bf16, out_bf16, ret_final;
};

// Workgroup id -> (b, h, chunk group).  Tiles are ordered (b, group, g, head
// in group) and dealt in contiguous runs to the 8 XCDs (workgroup n runs on
// XCD n % 8), so the heads that share one B/C group run side by side on one
// XCD and share its L2.
__device__ __forceinline__ bool decode_tile(const Params &p, int64_t ngroups_here, int64_t &b,
                                            int64_t &h, int64_t &j) {
  const int64_t total = p.batch * p.H * ngroups_here;
  const int64_t n = blockIdx.x;
  const int64_t per = (total + 7) / 8;
  const int64_t T = (n % 8) * per + n / 8;
  if (T >= total) return false;
  const int64_t hpg = p.H / p.G;
  const int64_t hh = T % hpg;
  int64_t rest = T / hpg;
  const int64_t g = rest % p.G;
  rest /= p.G;
  j = rest % ngroups_here;
  b = rest / ngroups_here;
  h = g * hpg + hh;
  return true;
}

// chunk_cumsum for one chunk: discretise dt (softplus, clamp), then the
// inclusive prefix of delta*A over the chunk, in log2 units.  Tokens past the
// sequence end get delta = 0, so they decay nothing and add nothing.
// Leaves Lam (log2) in sLam[0..Q) and delta in sDelta[0..Q); returns Lam_end.
template <int Q>
__device__ __forceinline__ float chunk_cumsum(const Params &p, int64_t b, int64_t h, int64_t t0,
                                              int Qc, float A2, float bias, float *sLam,
                                              float *sDelta, float *sWave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float a = 0.f, delta = 0.f;
  if (tid < Qc) {
    float u = p.dt[(b * p.L + t0 + tid) * p.H + h] + bias;
    if (p.dt_softplus) u = (u > 20.f) ? u : log1pf(expf(u));
    delta = fminf(fmaxf(u, p.dt_min), p.dt_max);
    a = delta * A2;
  }
  float v = a;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float nb = __shfl_up(v, off, 64);
    if (lane >= off) v += nb;
  }
  if (lane == 63) sWave[wave] = v;
  __syncthreads();
  float pre = 0.f;
  for (int w = 0; w < wave; ++w) pre += sWave[w];
  v += pre;
  if (tid < Q) {
    sLam[tid] = v;
    sDelta[tid] = delta;
  }
  __syncthreads();
  return sLam[Q - 1];
}

// Stage tokens [t0 + 64 jb, +64) of one chunk into LDS:
//   sB  [64][N]  B rows            (A operand of B.C^T; only if WANT_B)
//   sBT [N][64]  (w_j B_j)^T with w_j = exp(Lam_end - Lam_j) delta_j
//   sXT [P][64]  x^T
// Each thread loads 4 rows x 4 columns and transposes them in registers.
template <int N, bool F32, class IO, bool WANT_B>
__device__ __forceinline__ void stage_block(const Params &p, int64_t b, int64_t h, int64_t g,
                                            int64_t t0, int jb, int Qc, float lend2,
                                            const float *sLam, const float *sDelta,
                                            typename Mma<F32>::T *sB, typename Mma<F32>::T *sBT,
                                            typename Mma<F32>::T *sXT) {
  using T = typename Mma<F32>::T;
  using quad = typename Mma<F32>::quad;
  constexpr int LDN = N + 8, LDJ = kJB + 8;
  const int tid = threadIdx.x;
  // B block
  {
    constexpr int NG = N / 4;
    constexpr int RG = kThreads / NG;
    constexpr int PASSES = kJB / (4 * RG);
    const int ng = tid % NG, rg = tid / NG;
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int r0 = pass * 4 * RG + 4 * rg;
      f32x4 v[4];
      float wgt[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jl = kJB * jb + r0 + e;  // token within chunk
        if (jl < Qc) {
          v[e] = load4<IO>(p.B, ((b * p.L + t0 + jl) * p.G + g) * N + 4 * ng);
          wgt[e] = fast_exp2(lend2 - sLam[jl]) * sDelta[jl];
        } else {
          v[e] = f32x4{0.f, 0.f, 0.f, 0.f};
          wgt[e] = 0.f;
        }
        if (WANT_B) {
          quad q;
#pragma unroll
          for (int c = 0; c < 4; ++c) q[c] = (T)v[e][c];
          *reinterpret_cast<quad *>(&sB[(r0 + e) * LDN + 4 * ng]) = q;
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        quad q;
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = (T)(wgt[e] * v[e][c]);
        *reinterpret_cast<quad *>(&sBT[(4 * ng + c) * LDJ + r0]) = q;
      }
    }
  }
  // x block
  {
    constexpr int PG = kP / 4;  // 16
    const int pg = tid % PG, rg = tid / PG;  // rg in [0,16): rows 4rg..4rg+3
    const int r0 = 4 * rg;
    f32x4 v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jl = kJB * jb + r0 + e;
      v[e] = (jl < Qc) ? load4<IO>(p.x, ((b * p.L + t0 + jl) * p.H + h) * kP + 4 * pg)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      quad q;
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = (T)v[e][c];
      *reinterpret_cast<quad *>(&sXT[(4 * pg + c) * LDJ + r0]) = q;
    }
  }
}

// chunk_state on one staged block: wave w owns state rows p in [16w, 16w+16)
// and all N columns; S += X^T diag(w) B over the block's 64 tokens.
template <int N, bool F32>
__device__ __forceinline__ void state_block_mma(const typename Mma<F32>::T *sXT,
                                                const typename Mma<F32>::T *sBT, f32x4 *sacc) {
  using frag = typename Mma<F32>::frag;
  constexpr int LDJ = kJB + 8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < kJB / 32; ++kb) {
    const frag a = *reinterpret_cast<const frag *>(&sXT[(16 * w + lr) * LDJ + 32 * kb + 8 * lq]);
#pragma unroll
    for (int nt = 0; nt < N / 16; ++nt) {
      const frag bf = *reinterpret_cast<const frag *>(&sBT[(16 * nt + lr) * LDJ + 32 * kb + 8 * lq]);
      sacc[nt] = mma(a, bf, sacc[nt]);
    }
  }
}

// Row tiles (16 rows each) of a chunk owned by wave w.  With 8 or more tiles
// a wave takes mirrored pairs (w, 7-w) of every 8, balancing the causal work.
template <int Q>
__device__ __forceinline__ int row_tile(int k, int w) {
  constexpr int NT = Q / 16;
  if (NT == 4) return w;
  const int pi = k >> 1;
  return (k & 1) ? 8 * pi + 7 - w : 8 * pi + w;
}

// ---------------------------------------------------------------- kernels

// First pass (only when a sequence is split into several chunk groups): the
// state each of the first ngroups-1 groups builds from a zero start, and the
// group's total decay.
template <int Q, int N, bool F32, class IO>
__global__ __launch_bounds__(kThreads) void ssd_group_state_kernel(Params p) {
  using T = typename Mma<F32>::T;
  constexpr int LDJ = kJB + 8;
  __shared__ __attribute__((aligned(16))) T sBT[N * LDJ];
  __shared__ __attribute__((aligned(16))) T sXT[kP * LDJ];
  __shared__ float sLam[Q], sDelta[Q], sWave[4];

  int64_t b, h, j;
  if (!decode_tile(p, p.ngroups - 1, b, h, j)) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, lq = lane >> 4;
  const int64_t g = h / (p.H / p.G);
  const float A2 = p.A[h] * kLog2e;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.f;

  f32x4 sacc[N / 16];
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt) sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lgrp = 0.f;
  const int64_t c_begin = j * p.cpg, c_end = c_begin + p.cpg;  // never the last group
  for (int64_t c = c_begin; c < c_end; ++c) {
    const int64_t t0 = c * Q;
    const int Qc = (int)((p.L - t0) < Q ? (p.L - t0) : Q);
    const float lend2 = chunk_cumsum<Q>(p, b, h, t0, Qc, A2, bias, sLam, sDelta, sWave);
    const float dec = fast_exp2(lend2);
#pragma unroll
    for (int nt = 0; nt < N / 16; ++nt) sacc[nt] *= dec;
    lgrp += lend2;
    for (int jb = 0; jb < Q / kJB; ++jb) {
      if (kJB * jb >= Qc) break;
      __syncthreads();
      stage_block<N, F32, IO, false>(p, b, h, g, t0, jb, Qc, lend2, sLam, sDelta, nullptr, sBT, sXT);
      __syncthreads();
      state_block_mma<N, F32>(sXT, sBT, sacc);
    }
  }
  const int64_t slot = (b * p.H + h) * (p.ngroups - 1) + j;
  float *dst = p.grp_state + slot * (int64_t)(kP * N);
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(16 * w + 4 * lq + r) * N + 16 * nt + lr] = sacc[nt][r];
  if (threadIdx.x == 0) p.grp_lam[slot] = lgrp;
}

// state_passing across chunk groups (elementwise over P*N, sequential over
// groups): S = exp(Lam_grp) S + S_grp; slot j is overwritten with the state
// entering group j+1.
__global__ __launch_bounds__(kThreads) void ssd_group_passing_kernel(Params p, int PN) {
  const int64_t blocks_per_bh = PN / kThreads;
  const int64_t bh = blockIdx.x / blocks_per_bh;
  const int64_t e = (blockIdx.x % blocks_per_bh) * kThreads + threadIdx.x;
  float S = p.h0 ? p.h0[bh * PN + e] : 0.f;
  const int64_t ng1 = p.ngroups - 1;
  for (int64_t jj = 0; jj < ng1; ++jj) {
    const int64_t slot = bh * ng1 + jj;
    S = fast_exp2(p.grp_lam[slot]) * S + p.grp_state[slot * PN + e];
    p.grp_state[slot * PN + e] = S;
  }
}

// Main pass: chunk_scan over the chunks of one group, carrying the state.
template <int Q, int N, bool F32, class IO>
__global__ __launch_bounds__(kThreads) void ssd_chunk_scan_kernel(Params p) {
  using T = typename Mma<F32>::T;
  using frag = typename Mma<F32>::frag;
  using quad = typename Mma<F32>::quad;
  constexpr int NT = Q / 16;
  constexpr int NR = (NT >= 4) ? NT / 4 : 1;  // row tiles per wave
  constexpr int KB = N / 32;                  // K blocks over the state dim
  constexpr int LDN = N + 8, LDJ = kJB + 8;
  __shared__ __attribute__((aligned(16))) T sB[kJB * LDN];
  __shared__ __attribute__((aligned(16))) T sBT[N * LDJ];
  __shared__ __attribute__((aligned(16))) T sXT[kP * LDJ];
  __shared__ __attribute__((aligned(16))) T sS[kP * LDN];
  __shared__ float sLam[Q], sDelta[Q], sWave[4];

  int64_t b, h, j;
  if (!decode_tile(p, p.ngroups, b, h, j)) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, lq = lane >> 4;
  const int64_t g = h / (p.H / p.G);
  const float A2 = p.A[h] * kLog2e;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.f;
  const float Dh = p.D ? p.D[h] : 0.f;
  const int64_t bh = b * p.H + h;

  // state entering this group: h0 / zero for the first, the chained group
  // state otherwise.  Wave w holds rows [16w, 16w+16), in accumulator layout.
  f32x4 sacc[N / 16];
  {
    const float *init = (j == 0) ? (p.h0 ? p.h0 + bh * (int64_t)(kP * N) : nullptr)
                                 : p.grp_state + (bh * (p.ngroups - 1) + (j - 1)) * (int64_t)(kP * N);
#pragma unroll
    for (int nt = 0; nt < N / 16; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * w + 4 * lq + r, col = 16 * nt + lr;
        sacc[nt][r] = init ? init[row * N + col] : 0.f;
        sS[row * LDN + col] = (T)sacc[nt][r];
      }
  }

  const int64_t c_begin = j * p.cpg;
  const int64_t c_end = (c_begin + p.cpg < p.nc) ? c_begin + p.cpg : p.nc;
  for (int64_t c = c_begin; c < c_end; ++c) {
    const int64_t t0 = c * Q;
    const int Qc = (int)((p.L - t0) < Q ? (p.L - t0) : Q);
    const float lend2 = chunk_cumsum<Q>(p, b, h, t0, Qc, A2, bias, sLam, sDelta, sWave);

    // C rows of this wave's tiles, in registers (B operand of B.C^T and A
    // operand of C.S^T share one layout).
    frag cfr[NR][KB];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int i = 16 * row_tile<Q>(k, w) + lr;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (i < Qc) {
          cfr[k][kb] = load8<IO, F32>(p.C, ((b * p.L + t0 + i) * p.G + g) * N + 32 * kb + 8 * lq);
        } else {
#pragma unroll
          for (int s = 0; s < 8; ++s) cfr[k][kb][s] = (T)0.f;
        }
      }
    }

    // inter-chunk term: Y = diag(exp(Lam)) C S_in^T
    f32x4 yacc[NR][kP / 16];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int row0 = 16 * row_tile<Q>(k, w);
      float escale[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) escale[r] = fast_exp2(sLam[row0 + 4 * lq + r]);
#pragma unroll
      for (int pt = 0; pt < kP / 16; ++pt) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const frag sf = *reinterpret_cast<const frag *>(&sS[(16 * pt + lr) * LDN + 32 * kb + 8 * lq]);
          acc = mma(cfr[k][kb], sf, acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= escale[r];
        yacc[k][pt] = acc;
      }
    }

    // carried state: S <- exp(Lam_end) S, then += this chunk's S_loc below
    {
      const float dec = fast_exp2(lend2);
#pragma unroll
      for (int nt = 0; nt < N / 16; ++nt) sacc[nt] *= dec;
    }

    for (int jb = 0; jb < Q / kJB; ++jb) {
      if (kJB * jb >= Qc) break;
      __syncthreads();
      stage_block<N, F32, IO, true>(p, b, h, g, t0, jb, Qc, lend2, sLam, sDelta, sB, sBT, sXT);
      __syncthreads();
      // intra-chunk term for this wave's row tiles against tokens of block jb
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const int rt = row_tile<Q>(k, w);
        if (16 * rt + 15 < kJB * jb) continue;
        const int i = 16 * rt + lr;
        const float li = sLam[i];
#pragma unroll
        for (int js = 0; js < kJB / 32; ++js) {
          const int jbase = kJB * jb + 32 * js;
          if (jbase > 16 * rt + 15) break;
          // G^T[j][i] = B_j . C_i for j in [jbase, jbase+32), two 16x16 tiles
          f32x4 g0 = f32x4{0.f, 0.f, 0.f, 0.f}, g1 = g0;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const frag a0 = *reinterpret_cast<const frag *>(&sB[(32 * js + lr) * LDN + 32 * kb + 8 * lq]);
            const frag a1 = *reinterpret_cast<const frag *>(&sB[(32 * js + 16 + lr) * LDN + 32 * kb + 8 * lq]);
            g0 = mma(a0, cfr[k][kb], g0);
            g1 = mma(a1, cfr[k][kb], g1);
          }
          // M[i][j] = G[i][j] exp(Lam_i - Lam_j) delta_j (j <= i), held as the
          // A operand of M.X: lane keeps row i, K slots j = jbase+4lq+r and
          // jbase+16+4lq+r.
          frag mf;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int ja = jbase + 4 * lq + r, jc = ja + 16;
            const float ma = g0[r] * fast_exp2(li - sLam[ja]) * sDelta[ja];
            const float mc = g1[r] * fast_exp2(li - sLam[jc]) * sDelta[jc];
            mf[r] = (T)(ja <= i ? ma : 0.f);
            mf[4 + r] = (T)(jc <= i ? mc : 0.f);
          }
#pragma unroll
          for (int pt = 0; pt < kP / 16; ++pt) {
            const T *xrow = &sXT[(16 * pt + lr) * LDJ + 32 * js + 4 * lq];
            const quad lo = *reinterpret_cast<const quad *>(xrow);
            const quad hi = *reinterpret_cast<const quad *>(xrow + 16);
            frag xb;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              xb[s] = lo[s];
              xb[4 + s] = hi[s];
            }
            yacc[k][pt] = mma(mf, xb, yacc[k][pt]);
          }
        }
      }
      // chunk_state contribution of this block to the carried state
      state_block_mma<N, F32>(sXT, sBT, sacc);
    }

    // epilogue: + D x, gate, store
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int row0 = 16 * row_tile<Q>(k, w);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = row0 + 4 * lq + r;
        if (i >= Qc) continue;
        const int64_t base = ((b * p.L + t0 + i) * p.H + h) * kP;
#pragma unroll
        for (int pt = 0; pt < kP / 16; ++pt) {
          const int64_t idx = base + 16 * pt + lr;
          float y = yacc[k][pt][r];
          if (p.D) y += Dh * load1<IO>(p.x, idx);
          if (p.z) {
            const float zz = p.z_bf16 ? load1<IoBF16>(p.z, idx) : load1<IoF32>(p.z, idx);
            y *= zz / (1.f + expf(-zz));
          }
          if (p.out_bf16)
            static_cast<uint16_t *>(p.out)[idx] = f32_to_bf16_bits(y);
          else
            static_cast<float *>(p.out)[idx] = y;
        }
      }
    }

    // the state entering the next chunk, as the C.S^T operand
#pragma unroll
    for (int nt = 0; nt < N / 16; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sS[(16 * w + 4 * lq + r) * LDN + 16 * nt + lr] = (T)sacc[nt][r];
  }

  if (p.ret_final && j == p.ngroups - 1) {
    float *dst = p.final_state + bh * (int64_t)(kP * N);
#pragma unroll
    for (int nt = 0; nt < N / 16; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * w + 4 * lq + r) * N + 16 * nt + lr] = sacc[nt][r];
  }
}

// ---------------------------------------------------------------- host side

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool is_supported_chunk(int64_t q) { return q == 64 || q == 128 || q == 256; }

struct Plan {
  int64_t nc, cpg, ngroups;
  size_t state_bytes, lam_bytes;
};

// Validation of everything but pointers.
ssd_status check_shape(const ssd_desc *d, int64_t chunk) {
  if (!d) return SSD_ERR_INVALID_ARG;
  if (d->batch < 1 || d->seqlen < 1 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
      d->ngroups < 1 || chunk < 1)
    return SSD_ERR_INVALID_ARG;
  if (d->nheads % d->ngroups != 0) return SSD_ERR_INVALID_ARG;
  if (d->x_dtype != SSD_F32 && d->x_dtype != SSD_BF16 && d->x_dtype != SSD_F16)
    return SSD_ERR_INVALID_ARG;
  if (d->z_dtype != SSD_F32 && d->z_dtype != SSD_BF16 && d->z_dtype != SSD_F16)
    return SSD_ERR_INVALID_ARG;
  if (d->out_dtype != SSD_F32 && d->out_dtype != SSD_BF16 && d->out_dtype != SSD_F16)
    return SSD_ERR_INVALID_ARG;
  if (d->mma != SSD_MMA_F16 && d->mma != SSD_MMA_F32) return SSD_ERR_INVALID_ARG;
  if (d->chunks_per_wg < 0 || d->reserved != 0) return SSD_ERR_INVALID_ARG;
  if (!(d->dt_min <= d->dt_max)) return SSD_ERR_INVALID_ARG;  // also rejects NaN
  if (d->x_dtype == SSD_F16 || d->z_dtype == SSD_F16 || d->out_dtype == SSD_F16)
    return SSD_ERR_UNSUPPORTED;
  if (d->headdim != kP) return SSD_ERR_UNSUPPORTED;
  if (d->dstate != 64 && d->dstate != 128) return SSD_ERR_UNSUPPORTED;
  if (!is_supported_chunk(chunk)) return SSD_ERR_UNSUPPORTED;
  // 32-bit grid and 64-bit index headroom
  if (d->batch > (1 << 20) || d->nheads > (1 << 20) || d->seqlen > ((int64_t)1 << 31))
    return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

// Workgroups the plan aims for: two per CU on a 256-CU MI355X.
constexpr int64_t kTargetWorkgroups = 512;

Plan make_plan(const ssd_desc *d, int64_t chunk) {
  Plan pl;
  pl.nc = (d->seqlen + chunk - 1) / chunk;
  const int64_t bh = d->batch * d->nheads;
  int64_t cpg;
  if (d->chunks_per_wg > 0) {
    cpg = d->chunks_per_wg;
  } else if (bh >= kTargetWorkgroups) {
    cpg = pl.nc;
  } else {
    const int64_t want = (kTargetWorkgroups + bh - 1) / bh;
    cpg = pl.nc / want;
  }
  if (cpg < 1) cpg = 1;
  if (cpg > pl.nc) cpg = pl.nc;
  pl.cpg = cpg;
  pl.ngroups = (pl.nc + cpg - 1) / cpg;
  const int64_t slots = bh * (pl.ngroups - 1);
  pl.state_bytes = align_up((size_t)slots * (size_t)(d->headdim * d->dstate) * sizeof(float));
  pl.lam_bytes = align_up((size_t)slots * sizeof(float));
  if (slots == 0) pl.state_bytes = pl.lam_bytes = 0;
  return pl;
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

template <int Q, int N, bool F32, class IO>
ssd_status launch_all(const Params &prm, const Plan &pl, hipStream_t stream, const ssd_desc *d) {
  const int64_t bh = prm.batch * prm.H;
  if (pl.ngroups > 1) {
    const int64_t t1 = bh * (pl.ngroups - 1);
    const int64_t g1 = 8 * ((t1 + 7) / 8);
    hipLaunchKernelGGL((ssd_group_state_kernel<Q, N, F32, IO>), dim3((unsigned)g1), dim3(kThreads),
                       0, stream, prm);
    const int PN = kP * N;
    hipLaunchKernelGGL(ssd_group_passing_kernel, dim3((unsigned)(bh * (PN / kThreads))),
                       dim3(kThreads), 0, stream, prm, PN);
  }
  const int64_t t2 = bh * pl.ngroups;
  const int64_t g2 = 8 * ((t2 + 7) / 8);
  if (d->ev_main_begin && hipEventRecord(static_cast<hipEvent_t>(d->ev_main_begin), stream) != hipSuccess)
    return SSD_ERR_LAUNCH;
  hipLaunchKernelGGL((ssd_chunk_scan_kernel<Q, N, F32, IO>), dim3((unsigned)g2), dim3(kThreads), 0,
                     stream, prm);
  if (hipGetLastError() != hipSuccess) return SSD_ERR_LAUNCH;
  if (d->ev_main_end && hipEventRecord(static_cast<hipEvent_t>(d->ev_main_end), stream) != hipSuccess)
    return SSD_ERR_LAUNCH;
  return SSD_OK;
}

template <int Q, int N, bool F32>
ssd_status dispatch_io(const Params &prm, const Plan &pl, hipStream_t s, const ssd_desc *d) {
  if (d->x_dtype == SSD_BF16) return launch_all<Q, N, F32, IoBF16>(prm, pl, s, d);
  return launch_all<Q, N, F32, IoF32>(prm, pl, s, d);
}

template <int Q, int N>
ssd_status dispatch_mma(const Params &prm, const Plan &pl, hipStream_t s, const ssd_desc *d) {
  if (d->mma == SSD_MMA_F32) return dispatch_io<Q, N, true>(prm, pl, s, d);
  return dispatch_io<Q, N, false>(prm, pl, s, d);
}

template <int Q>
ssd_status dispatch_n(const Params &prm, const Plan &pl, hipStream_t s, const ssd_desc *d) {
  if (d->dstate == 64) return dispatch_mma<Q, 64>(prm, pl, s, d);
  return dispatch_mma<Q, 128>(prm, pl, s, d);
}

}  // namespace

extern "C" {

void ssd_desc_init(ssd_desc *d, int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, int64_t ngroups) {
  if (!d) return;
  memset(d, 0, sizeof(*d));
  d->batch = batch;
  d->seqlen = seqlen;
  d->nheads = nheads;
  d->headdim = headdim;
  d->dstate = dstate;
  d->ngroups = ngroups;
  d->x_dtype = SSD_F32;
  d->z_dtype = SSD_F32;
  d->out_dtype = SSD_F32;
  d->mma = SSD_MMA_F16;
  d->dt_min = 0.f;
  d->dt_max = INFINITY;
}

ssd_status ssd_fwd_workspace_size(const ssd_desc *d, int64_t chunk, size_t *bytes) {
  if (!bytes) return SSD_ERR_INVALID_ARG;
  const ssd_status st = check_shape(d, chunk);
  if (st != SSD_OK) return st;
  const Plan pl = make_plan(d, chunk);
  *bytes = pl.state_bytes + pl.lam_bytes;
  return SSD_OK;
}

ssd_status ssd_fwd_plan(const ssd_desc *d, int64_t chunk, int64_t *chunks_per_wg,
                        int64_t *n_chunk_groups) {
  const ssd_status st = check_shape(d, chunk);
  if (st != SSD_OK) return st;
  const Plan pl = make_plan(d, chunk);
  if (chunks_per_wg) *chunks_per_wg = pl.cpg;
  if (n_chunk_groups) *n_chunk_groups = pl.ngroups;
  return SSD_OK;
}

ssd_status ssd_fwd(const void *x, const float *dt, const float *A, const void *B, const void *C,
                   const float *D, int64_t chunk, int dt_softplus, int return_final_state,
                   void *out, float *final_state, void *stream, const ssd_desc *d) {
  const ssd_status st = check_shape(d, chunk);
  if (st != SSD_OK) return st;
  if (!x || !dt || !A || !B || !C || !out) return SSD_ERR_INVALID_ARG;
  if (return_final_state && !final_state) return SSD_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(out) ||
      (d->z && !aligned16(d->z)) || !aligned16(dt) ||
      (d->initial_state && !aligned16(d->initial_state)) ||
      (return_final_state && !aligned16(final_state)))
    return SSD_ERR_INVALID_ARG;
  const Plan pl = make_plan(d, chunk);
  const size_t need = pl.state_bytes + pl.lam_bytes;
  if (need > 0 && (!d->workspace || d->workspace_bytes < need || !aligned16(d->workspace)))
    return SSD_ERR_WORKSPACE;

  Params prm;
  memset(&prm, 0, sizeof(prm));
  prm.x = x;
  prm.dt = dt;
  prm.A = A;
  prm.B = B;
  prm.C = C;
  prm.D = D;
  prm.z = d->z;
  prm.dt_bias = d->dt_bias;
  prm.h0 = d->initial_state;
  prm.out = out;
  prm.final_state = final_state;
  prm.grp_state = need > 0 ? static_cast<float *>(d->workspace) : nullptr;
  prm.grp_lam = need > 0 ? reinterpret_cast<float *>(static_cast<char *>(d->workspace) + pl.state_bytes)
                         : nullptr;
  prm.batch = d->batch;
  prm.L = d->seqlen;
  prm.H = d->nheads;
  prm.G = d->ngroups;
  prm.nc = pl.nc;
  prm.ngroups = pl.ngroups;
  prm.cpg = pl.cpg;
  prm.dt_min = d->dt_min;
  prm.dt_max = d->dt_max;
  prm.dt_softplus = dt_softplus ? 1 : 0;
  prm.z_bf16 = d->z_dtype == SSD_BF16;
  prm.out_bf16 = d->out_dtype == SSD_BF16;
  prm.ret_final = return_final_state ? 1 : 0;

  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (chunk) {
    case 64: return dispatch_n<64>(prm, pl, s, d);
    case 128: return dispatch_n<128>(prm, pl, s, d);
    default: return dispatch_n<256>(prm, pl, s, d);
  }
}

const char *ssd_status_str(int status) {
  switch (status) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_INVALID_ARG: return "SSD_ERR_INVALID_ARG: invalid argument";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: shape or dtype not compiled";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
    case SSD_ERR_LAUNCH: return "SSD_ERR_LAUNCH: kernel launch failed";
    default: return "unknown ssd_status";
  }
}

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

}  // extern "C"
