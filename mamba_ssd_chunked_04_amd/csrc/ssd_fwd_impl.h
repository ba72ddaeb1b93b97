// Mamba-2 SSD chunked forward for MI355X (gfx950, CDNA4): the kernels and their
// launch templates (internal header; the C ABI of include/ssd_mi355x.h is
// in ssd_fwd.hip, and ssd_fwd_q{64,128,256}.hip instantiate the launches of
// one chunk size each, so the three compile in parallel).
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
//   * one workgroup (4 or 8 wave64s) walks `cpg` consecutive chunks of one
//     (b, h), keeping the P x N state in MFMA accumulators across chunks, so
//     the state recurrence costs no HBM traffic inside a chunk group;
//   * chunk_cumsum runs inside the matrix passes, at the start of each chunk;
//   * when (b, h) pairs alone cannot fill 256 CUs, the sequence is cut into
//     chunk groups: a first pass (ssd_group_state_kernel) builds each
//     group's state from zero, and the main pass (ssd_chunk_scan_kernel)
//     chains the aggregates of the groups before its own (state_passing)
//     to start every group from its entering state (with many groups a
//     separate elementwise pass, ssd_group_passing_kernel, chains them once);
//   * all contractions (C.B^T, M.X, C.S^T, X^T.diag(w).B) are
//     v_mfma_f32_16x16x32_f16 tiles (or 16x16x4 fp32 on the check path) with
//     B, X staged in LDS 64 tokens at a time and C held in registers;
//   * the masked C.B^T block is computed transposed, so its accumulator
//     layout is directly the A operand of the M.X product (no LDS round trip);
//   * workgroup ids are swizzled so heads sharing a B/C group run on the same
//     XCD (shared L2);
//   * packed variable-length sequences (cu_seqlens) are batch rows whose
//     token span comes from the offsets: each is chunked from its own start
//     and its state restarts there, the form page "Mamba-2 SSD for Ascend
//     NPU" lists under "Limitations and roadmap" (varlen, cu_seqlens).
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/ssd_mi355x.h"

namespace ssd_fwd_impl {

constexpr int kJB = 64;         // tokens per LDS-staged block
constexpr int kP = 64;          // compiled head dim
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- operand types
// Matrix-core operand precision (the descriptor's ssd_mma): fp16 or bf16
// operands with fp32 accumulation, or fp32 throughout (the check path).
constexpr int kMmaF16 = 0, kMmaBF16 = 1, kMmaF32 = 2;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
template <int MM> struct Mma;
template <> struct Mma<kMmaF16> {
  using T = _Float16;
  using frag = f16x8;
  using quad = f16x4;
};
template <> struct Mma<kMmaBF16> {
  using T = __bf16;
  using frag = bf16x8;
  using quad = bf16x4;
};
template <> struct Mma<kMmaF32> {
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
__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8 &a, const f32x8 &b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 8; ++s)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// Two floats rounded to the operand type E as one packed conversion
// (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32 on gfx950, round to nearest even;
// for E = float a copy).
template <class E> struct Pair2 { E x, y; };
template <class E>
__device__ __forceinline__ Pair2<E> cvt2(float a, float b) {
  if constexpr (sizeof(E) == 4) {
    return {a, b};
  } else {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef E e2 __attribute__((ext_vector_type(2)));
    const e2 v = __builtin_convertvector((f2){a, b}, e2);
    return {v.x, v.y};
  }
}

// softplus(u) = max(u, 0) + log1p(e) with e = exp(-|u|) in (0, 1], without
// the library log1p (about 70 instructions).  Below 1/16, log1p(e) is its
// alternating series to e^5 (truncation below e^6/6, under 1.7e-7 of the
// result); from 1/16 on, the hardware log2 of v = 1 + e times ln 2, with the
// rounding of v undone by the factor e / (v - 1) (v - 1 is exact), so the
// result keeps a few ulp where the plain log of 1 + e would lose the digits
// of a small e.
__device__ __forceinline__ float softplus_f(float u) {
  const float e = __expf(-fabsf(u));
  const float v = 1.f + e;
  const float big = __builtin_amdgcn_logf(v) * 0.6931471805599453f *
                    (e * __builtin_amdgcn_rcpf(v - 1.f));
  const float small = e * (1.f - e * (0.5f - e * (1.f / 3.f - e * (0.25f - e * 0.2f))));
  return fmaxf(u, 0.f) + (e < 0.0625f ? small : big);
}

// ---------------------------------------------------------------- buffer access
// Every tensor of one batch row is addressed through a raw buffer resource
// (base in SGPRs, 32-bit byte offsets per lane).  The hardware range check
// returns zeros for loads past the end of the row's data and drops stores
// past it, which is how tokens beyond the sequence end are handled.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Cache-policy bit of buffer operations for device scope: such a store is
// written through its XCD's L2 (visible to every XCD once complete, and
// left clean, so a kernel's end has less to write back), such a load reads
// past it.
constexpr int kSc1 = 16;

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

// Storage formats of x, B, C (and z).  Loads are split into an issue step
// (raw registers) and a convert step so a whole block's loads can be in
// flight before any of them is used.  Offsets are in elements.
struct IoF32 {
  static constexpr int esz = 4;
  using raw4 = f32x4;
  struct raw8 {
    f32x4 lo, hi;
  };
  static __device__ __forceinline__ raw4 load4(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off * 4, 0, 0));
  }
  static __device__ __forceinline__ raw8 load8(rsrc_t r, uint32_t off) {
    return raw8{load4(r, off), load4(r, off + 4)};
  }
  static __device__ __forceinline__ f32x4 cvt4(const raw4 &v) { return v; }
  static __device__ __forceinline__ float cvt8(const raw8 &v, int e) {
    return e < 4 ? v.lo[e] : v.hi[e - 4];
  }
  static __device__ __forceinline__ float load1(rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off * 4, 0, 0));
  }
  typedef float raw2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ raw2 load2(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(raw2, __builtin_amdgcn_raw_buffer_load_b64(r, off * 4, 0, 0));
  }
  static __device__ __forceinline__ float cvt2(const raw2 &v, int e) { return v[e]; }
};

struct IoBF16 {
  static constexpr int esz = 2;
  typedef unsigned int raw4 __attribute__((vector_size(8)));
  typedef unsigned int raw8 __attribute__((vector_size(16)));
  static __device__ __forceinline__ raw4 load4(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off * 2, 0, 0);
  }
  static __device__ __forceinline__ raw8 load8(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off * 2, 0, 0);
  }
  static __device__ __forceinline__ f32x4 cvt4(const raw4 &v) {
    f32x4 o;
    o[0] = bf16_bits_to_f32(v[0] & 0xffffu);
    o[1] = bf16_bits_to_f32(v[0] >> 16);
    o[2] = bf16_bits_to_f32(v[1] & 0xffffu);
    o[3] = bf16_bits_to_f32(v[1] >> 16);
    return o;
  }
  static __device__ __forceinline__ float cvt8(const raw8 &v, int e) {
    const uint32_t w = v[e >> 1];
    return bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xffffu));
  }
  static __device__ __forceinline__ float load1(rsrc_t r, uint32_t off) {
    return bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off * 2, 0, 0));
  }
  typedef uint32_t raw2;
  static __device__ __forceinline__ raw2 load2(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off * 2, 0, 0);
  }
  static __device__ __forceinline__ float cvt2(const raw2 &v, int e) {
    return bf16_bits_to_f32(e ? (v >> 16) : (v & 0xffffu));
  }
};

// Storage formats of x and of B/C (which may differ).
template <class IX, class IB> struct IoPair {
  using X = IX;
  using BC = IB;
};

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
  float *grp_state;  // [B*H][ngroups-1][P*N]: group aggregates (state from a zero
                     // start), or entering states once the passing pass ran
  float *grp_lam;    // [B*H][ngroups-1]: group total log2-decay
  const int32_t *cu_seqlens;  // packed calls: [batch+1] token offsets, else NULL
  int32_t *error_flag;        // packed calls: set to 1 on offsets that break the contract
  int64_t packed_tokens;      // packed calls: T when known (offsets are clamped to it), else 0
  int64_t xs, bs, zs, dts;    // elements between consecutive tokens of x, B/C, z, dt
  int64_t batch, L, H, G, nc, ngroups, cpg;
  int Q;
  float dt_min, dt_max;
  int dt_softplus, z_bf16, out_bf16, ret_final;
  int chained;  // grp_state holds entering states (the passing pass ran)
  // fused gated RMSNorm epilogue (norm_w != NULL): groups of norm_k heads,
  // exchanged per chunk through norm_rec [B][nchk_row][H][Q] (per-token
  // partial sums of squares, each with the call's tag) and norm_sync (the
  // epoch the tags derive from, and the count of finished workgroups)
  const float *norm_w;
  uint64_t *norm_rec;
  uint64_t *norm_sync;
  int64_t nchk_row;
  float norm_eps;
  int norm_k;
};

// Quotient and remainder of non-negative values below 2^32 (tile indices,
// head, group and chunk counts): the 32-bit sequence is a fraction of the
// 64-bit one, and these sit before a workgroup's first loads.
__device__ __forceinline__ int64_t udiv32(int64_t a, int64_t b) {
  return (int64_t)((uint32_t)a / (uint32_t)b);
}
__device__ __forceinline__ int64_t umod32(int64_t a, int64_t b) {
  return (int64_t)((uint32_t)a % (uint32_t)b);
}

// Workgroup id -> (b, h, chunk group).  Tiles are ordered (b, group, g, head
// in group); workgroup n runs on XCD n % 8.  Dense calls deal the tiles in
// contiguous runs to the XCDs, so the heads that share one B/C group run side
// by side on one XCD and share its L2.  Packed calls, whose rows differ in
// length, deal units of those heads round-robin over the XCDs instead (unit
// u on XCD u % 8), so long and short sequences spread over all of them; the
// grid then has 8 * hpg * ceil(units / 8) workgroups (tile_grid).  With
// `late_first` the chunk groups are dealt from the last one down (later
// groups have more to do before their first chunk): when the main pass
// folds an even number of groups itself, a dense call's late group ng-1-i is
// dealt with its early partner i on one XCD, late members first, so each XCD
// holds the same mix of long and short prologues and a CU's two workgroups
// tend to be such a pair (headline main pass 39.4 -> 38.3 us).  (The
// packed and the plain dense decode keep 64-bit divisions: with udiv32 there
// the compiler spilled scalar registers inside the block loop of the
// 256-token gated kernel, 1% slower.)
__device__ __forceinline__ bool decode_tile(const Params &p, int64_t ngroups_here, int64_t &b,
                                            int64_t &h, int64_t &j, bool late_first = false) {
  const int64_t total = p.batch * p.H * ngroups_here;
  const int64_t n = blockIdx.x;
  const int64_t hpg = p.H / p.G;
  int64_t T;
  if (p.cu_seqlens) {
    const int64_t k = n / 8;
    T = ((k / hpg) * 8 + n % 8) * hpg + k % hpg;
  } else if (late_first && ngroups_here % 2 == 0 && !p.chained) {
    // tiles paired, late group ng-1-i with early group i (same b, g and
    // head), in the order (b, i, g, head in group); each XCD takes a
    // contiguous run of pairs and dispatches its late members first, then
    // the early ones in the same order (tile_grid workgroups)
    const int64_t pairs = total / 2, pp = (pairs + 7) / 8;
    const int64_t k = n / 8, half = udiv32(k, pp), pr = (n % 8) * pp + umod32(k, pp);
    if (half > 1 || pr >= pairs) return false;
    const int64_t hh = umod32(pr, hpg);
    int64_t rest = udiv32(pr, hpg);
    const int64_t g = umod32(rest, p.G);
    rest = udiv32(rest, p.G);
    const int64_t i = umod32(rest, ngroups_here / 2);
    b = udiv32(rest, ngroups_here / 2);
    j = half == 0 ? ngroups_here - 1 - i : i;
    h = g * hpg + hh;
    return true;
  } else {
    const int64_t per = (total + 7) / 8;
    T = (n % 8) * per + n / 8;
  }
  if (T >= total) return false;
  const int64_t hh = T % hpg;
  int64_t rest = T / hpg;
  const int64_t g = rest % p.G;
  rest /= p.G;
  j = rest % ngroups_here;
  if (late_first) j = ngroups_here - 1 - j;
  b = rest / ngroups_here;
  h = g * hpg + hh;
  return true;
}

// Tokens of batch row b: [start, start + len) on the token axis.  Dense
// calls: b*L and L.  Packed calls: the row is sequence b of cu_seqlens,
// with its offsets clamped to [0, T] (when T is known) and its length to
// [0, L] (L is then the longest sequence, which the plan is made for), so
// that malformed offsets never address memory outside x, B, C and out; the
// main pass reports them through error_flag (offsets_break_contract).
struct RowSpan {
  int64_t start, len;
};

__device__ __forceinline__ RowSpan row_span(const Params &p, int64_t b) {
  if (!p.cu_seqlens) return {b * p.L, p.L};
  int64_t s = p.cu_seqlens[b], e = p.cu_seqlens[b + 1];
  s = s < 0 ? 0 : s;
  if (p.packed_tokens > 0) {
    s = s > p.packed_tokens ? p.packed_tokens : s;
    e = e > p.packed_tokens ? p.packed_tokens : e;
  }
  const int64_t len = e - s;
  return {s, len < 0 ? 0 : (len > p.L ? p.L : len)};
}

// Whether the offsets of packed row b break the contract of the call: a
// sequence longer than L, decreasing offsets, a negative offset or one past
// T (when T is known).
__device__ __forceinline__ bool offsets_break_contract(const Params &p, int64_t b) {
  const int64_t s = p.cu_seqlens[b], e = p.cu_seqlens[b + 1];
  return s < 0 || e < s || e - s > p.L || (p.packed_tokens > 0 && e > p.packed_tokens);
}

// Chunks of a row and the chunk groups that hold them; an empty row keeps
// one group, which writes its final state (the initial state).
__device__ __forceinline__ int64_t row_chunks(const Params &p, int64_t len) {
  return udiv32(len + p.Q - 1, p.Q);
}
__device__ __forceinline__ int64_t row_groups(const Params &p, int64_t len) {
  const int64_t ng = udiv32(row_chunks(p, len) + p.cpg - 1, p.cpg);
  return ng < 1 ? 1 : ng;
}

// Buffer resources and element offsets of one (b, h) sequence.  Tokens of
// x, B/C (and z, dt) are xs, bs (zs, dts) elements apart: the dense layouts
// [.., H, P] and [.., G, N] or strided views of wider token-major rows (such
// as a conv output holding x, B and C side by side).  out is always dense.
template <int N, class IO>
struct SeqView {
  rsrc_t x, B, C;
  uint32_t H, G, h, g, xs, bs, dts;
  __device__ __forceinline__ SeqView(const Params &p, const RowSpan &rs, int64_t h_, int64_t g_) {
    const uint64_t L = (uint64_t)rs.len, t0 = (uint64_t)rs.start;
    H = (uint32_t)p.H;
    G = (uint32_t)p.G;
    h = (uint32_t)h_;
    g = (uint32_t)g_;
    xs = (uint32_t)p.xs;
    bs = (uint32_t)p.bs;
    dts = (uint32_t)p.dts;
    constexpr int xe = IO::X::esz, be = IO::BC::esz;
    x = make_rsrc(static_cast<const char *>(p.x) + t0 * p.xs * xe, (uint32_t)(L * p.xs * xe));
    B = make_rsrc(static_cast<const char *>(p.B) + t0 * p.bs * be, (uint32_t)(L * p.bs * be));
    C = make_rsrc(static_cast<const char *>(p.C) + t0 * p.bs * be, (uint32_t)(L * p.bs * be));
  }
  __device__ __forceinline__ uint32_t xoff(uint32_t t, uint32_t col) const { return t * xs + h * kP + col; }
  __device__ __forceinline__ uint32_t boff(uint32_t t, uint32_t col) const { return t * bs + g * N + col; }
  // dense [.., H, P] offset (out)
  __device__ __forceinline__ uint32_t ooff(uint32_t t, uint32_t col) const { return (t * H + h) * kP + col; }
};

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, then synchronises the workgroup.  Unlike __syncthreads it does
// not drain outstanding global loads, so prefetched data stays in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Per-chunk scalars in LDS (Lam in log2 units).
//   lam[j]   inclusive in-chunk prefix of delta*A;  delta[j]
//   w[j]     exp(Lam_end - Lam_j) delta_j      (chunk_state weights)
//   u[j]     exp(Lam_m - Lam_j) delta_j, m the reference token (16th) of j's
//            32-token sub-block; mid[j/32] = Lam_m
//   dts[j]   raw dt of token j, staged one chunk ahead
// (16-byte aligned, size a multiple of 16: the second buffer of a pair keeps
// the 16-byte alignment of the f32x4 reads of lam and u)
template <int Q> struct alignas(16) ChunkLds {
  float lam[Q], delta[Q], w[Q], u[Q], dts[Q], mid[Q / 32];
  float lend;  // Lam_end and the factored flag, when only the writing waves
  int fac;     // prepare the chunk (chunk_prep with ONCE)
};

// chunk_cumsum inside the matrix passes.  The raw dt of a chunk is loaded
// two chunks ahead, one token per thread, and staged in the chunk's LDS
// scalars one chunk ahead.  Lane l of every wave then takes the tokens
// l + 64 m of the chunk (m < Q/64) and computes, redundantly in each wave,
// delta = clamp(softplus(dt + dt_bias)) (0 past the sequence end) and the
// inclusive in-chunk prefix Lam of delta*A in log2 units (a wavefront scan
// per 64 tokens plus the running total of the earlier ones).
// Thread t < Q handles token t; threads past Q load token Q-1 again (one
// merged request per wave) and store that same value over it, which keeps
// the load and the LDS store free of branches (a branch here makes the
// compiler wait for every load in flight).
__device__ __forceinline__ uint32_t dt_token(int Q, uint32_t tid) {
  return tid < (uint32_t)Q ? tid : (uint32_t)Q - 1;
}
__device__ __forceinline__ uint32_t dt_token(int Q) { return dt_token(Q, threadIdx.x); }

// raw dt of token t0 + dt_token (dt tokens dts elements apart)
__device__ __forceinline__ float load_dt(rsrc_t rdt, uint32_t dts, uint32_t h, uint32_t t0, int Q,
                                         uint32_t tid) {
  return __uint_as_float(
      __builtin_amdgcn_raw_buffer_load_b32(rdt, ((t0 + dt_token(Q, tid)) * dts + h) * 4, 0, 0));
}
__device__ __forceinline__ float load_dt(rsrc_t rdt, uint32_t dts, uint32_t h, uint32_t t0, int Q) {
  return load_dt(rdt, dts, h, t0, Q, threadIdx.x);
}

template <int Q>
__device__ __forceinline__ void stage_dt(float v, ChunkLds<Q> &cl, uint32_t tid) {
  cl.dts[dt_token(Q, tid)] = v;
}
template <int Q>
__device__ __forceinline__ void stage_dt(float v, ChunkLds<Q> &cl) {
  stage_dt<Q>(v, cl, threadIdx.x);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves:
// shifts by 1, 2, 4, 8 inside each row of 16 lanes, then row 0's total added
// to row 1 and row 2's to row 3 (row_bcast:15), then rows 0-1's total to
// rows 2-3 (row_bcast:31).  Lanes a move does not reach add zero.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  int t;
  const int x = __float_as_int(v);
  switch (ctrl_sel) {
    case 0: t = __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true); break;  // row_shr:1
    case 1: t = __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true); break;  // row_shr:2
    case 2: t = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true); break;  // row_shr:4
    case 3: t = __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true); break;  // row_shr:8
    case 4: t = __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false); break; // row_bcast:15
    default: t = __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false); break; // row_bcast:31
  }
  return v + __int_as_float(t);
}

__device__ __forceinline__ float wave_inclusive_sum(float v) {
#pragma unroll
  for (int k = 0; k < 6; ++k) v = dpp_add(v, k);
  return v;
}

// Discretise and scan the chunk starting at token t0, then fill its LDS
// scalars (the caller puts a barrier before any reader).  Returns Lam_end and
// whether |delta*A| <= 7 (log2 units) for every token, which keeps the
// factored intra-chunk decay of the main pass inside fp32 range.  With ONCE
// only the waves that write the records (w < Q/64) prepare the chunk and
// they also store Lam_end and the flag in the LDS scalars, where the other
// waves read them after the barrier (lend and factored are then left unset
// in those waves): in the main pass that frees the other waves' SIMDs
// (H256 1.190 -> 1.162 ms, long 0.185 -> 0.181 ms, gated 0.534 -> 0.526 ms).
template <int Q, bool ONCE = false>
__device__ __forceinline__ void chunk_prep(const Params &p, uint32_t t0, uint64_t len,
                                           float a_h, float bias, ChunkLds<Q> &cl, float &lend,
                                           bool &factored, int tid) {
  const int lane = tid & 63, w = tid >> 6;
  if (ONCE && w >= Q / 64) return;
  float lam[Q / 64], del[Q / 64];
  float run = 0.f;
  bool big = false;
#pragma unroll
  for (int m = 0; m < Q / 64; ++m) {
    float u = cl.dts[lane + 64 * m] + bias;
    // softplus as max(u, 0) + log1p(exp(-|u|)): no cancellation for negative
    // u (where log(1 + exp(u)) loses the digits of a small step) and no
    // overflow for large u; the backward uses the same form (with the
    // library log1p)
    if (p.dt_softplus) u = softplus_f(u);
    const float delta = (t0 + lane + 64 * m < len) ? fminf(fmaxf(u, p.dt_min), p.dt_max) : 0.f;
    const float a = delta * a_h * kLog2e;
    big |= fabsf(a) > 7.f;
    const float v = wave_inclusive_sum(a);
    lam[m] = v + run;
    del[m] = delta;
    run += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  }
  lend = run;
  factored = __ballot(big) == 0;
  if (ONCE && w == 0 && lane == 0) {
    cl.lend = lend;
    cl.fac = factored ? 1 : 0;
  }
  // wave w < Q/64 writes the records of tokens 64 w .. 64 w + 63
  if (w < Q / 64) {
    float lm = 0.f, dl = 0.f;
#pragma unroll
    for (int m = 0; m < Q / 64; ++m)
      if (m == w) {
        lm = lam[m];
        dl = del[m];
      }
    const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lm), 16));
    const float m1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lm), 48));
    const float mid = (lane < 32) ? m0 : m1;
    const int t = 64 * w + lane;
    cl.lam[t] = lm;
    cl.delta[t] = dl;
    cl.w[t] = fast_exp2(lend - lm) * dl;
    cl.u[t] = fast_exp2(mid - lm) * dl;
    if ((lane & 31) == 16) cl.mid[t >> 5] = lm;
  }
}
template <int Q, bool ONCE = false>
__device__ __forceinline__ void chunk_prep(const Params &p, uint32_t t0, uint64_t len,
                                           float a_h, float bias, ChunkLds<Q> &cl, float &lend,
                                           bool &factored) {
  chunk_prep<Q, ONCE>(p, t0, len, a_h, bias, cl, lend, factored, (int)threadIdx.x);
}

// Raw global data of one 64-token block: B rows [64][N] and x rows [64][P],
// spread over the workgroup's T threads in units of 4 rows x 4 columns.
template <int N, class IO, int T>
struct BlockRaw {
  static constexpr int NG = N / 4;                  // column groups of B
  static constexpr int UB = 16 * NG;                // B units
  // x units: 4 tokens x 4 columns, or 4 tokens x 2 columns when the
  // workgroup has at least twice as many threads as 4-column units (every
  // thread then holds one unit, in half the registers)
  static constexpr bool XPAIR = T >= 2 * 16 * (kP / 4);
  static constexpr int UX = XPAIR ? 16 * (kP / 2) : 16 * (kP / 4);
  static constexpr int KB_ = (UB + T - 1) / T;      // B units per thread
  static constexpr int KX = (UX + T - 1) / T;       // x units per thread
  typename IO::BC::raw4 b[KB_][4];
  typename IO::X::raw4 x[XPAIR ? 1 : KX][XPAIR ? 1 : 4];
  typename IO::X::raw2 x2[XPAIR ? KX : 1][XPAIR ? 4 : 1];
};

// Staging unit u -> (token quad rg in 0..15, column quad cg).  Every 64
// consecutive units cover an 8 x 8 tile of (rg, cg) pairs, so one wave's load
// of a row reads 8 column quads (a whole 128-byte line of fp32).  Inside each
// 16-unit group the pairs lie on a diagonal band: both the row-major writes
// (rows 4rg+e, 8-byte column quads) and the transposed writes (rows 4cg+c,
// 8-byte token quads) of the group then fall on 16 distinct LDS bank pairs
// (LDS writes serve 16 lanes of 8 bytes per cycle over 32 banks).
__device__ __forceinline__ void unit_of(int u, int &rg, int &cg) {
  const int i = u & 15, d = (u >> 4) & 3, t = u >> 6, q = i >> 2;
  rg = (i & 1) + 2 * q + 8 * (t & 1);
  cg = ((i >> 1) & 1) + 2 * ((q + d) & 3) + 8 * (t >> 1);
}

// Past-the-end element offset: the buffer range check turns a load from it
// into zeros (no memory access).  Every row buffer is below 2^31 bytes.
constexpr uint32_t kNoElem = 0x20000000u;

// Issue the loads of the 64-token block starting at token tb.  The loads are
// unconditional (units past the block's count read kNoElem) so that they stay
// in flight until the block is stored.
template <int N, class IO, int T>
__device__ __forceinline__ void load_block(const SeqView<N, IO> &sv, uint32_t tb,
                                           BlockRaw<N, IO, T> &r) {
  using BR = BlockRaw<N, IO, T>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < BR::KB_; ++k) {
    const int u = tid + T * k;
    const bool ok = BR::UB % T == 0 || u < BR::UB;
    int rg, ng;
    unit_of(u, rg, ng);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r.b[k][e] = IO::BC::load4(sv.B, ok ? sv.boff(tb + 4 * rg + e, 4 * ng) : kNoElem);
  }
#pragma unroll
  for (int k = 0; k < BR::KX; ++k) {
    const int u = tid + T * k;
    const bool ok = BR::UX % T == 0 || u < BR::UX;
    int rg, pg;
    unit_of(u, rg, pg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (BR::XPAIR)
        r.x2[k][e] = IO::X::load2(sv.x, ok ? sv.xoff(tb + 4 * rg + e, 2 * pg) : kNoElem);
      else
        r.x[k][e] = IO::X::load4(sv.x, ok ? sv.xoff(tb + 4 * rg + e, 4 * pg) : kNoElem);
    }
  }
}

// Write a loaded block into LDS in the MMA operand type:
//   sB  [64][N]  B rows            (A operand of B.C^T; only if WANT_B)
//   sBT [N][64]  (w_j B_j)^T
//   sXT [P][64]  x^T
template <int N, int MM, class IO, int T, bool WANT_B>
__device__ __forceinline__ void store_block(const BlockRaw<N, IO, T> &r, int jb, const float *sw,
                                            typename Mma<MM>::T *sB, typename Mma<MM>::T *sBT,
                                            typename Mma<MM>::T *sXT, bool want_bt = true) {
  using E = typename Mma<MM>::T;
  using quad = typename Mma<MM>::quad;
  using BR = BlockRaw<N, IO, T>;
  constexpr int LDN = N + 8, LDJ = kJB + 8;
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < BR::KB_; ++k) {
    const int u = tid + T * k;
    if (u < BR::UB) {
      int rg, ng;
      unit_of(u, rg, ng);
      const int r0 = 4 * rg;
      f32x4 v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = IO::BC::cvt4(r.b[k][e]);
        if (WANT_B) {
          quad q;
#pragma unroll
          for (int c = 0; c < 4; ++c) q[c] = (E)v[e][c];
          *reinterpret_cast<quad *>(&sB[(r0 + e) * LDN + 4 * ng]) = q;
        }
      }
      if (want_bt) {
        const f32x4 wgt = *reinterpret_cast<const f32x4 *>(&sw[kJB * jb + r0]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          quad q;
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = (E)(wgt[e] * v[e][c]);
          *reinterpret_cast<quad *>(&sBT[(4 * ng + c) * LDJ + r0]) = q;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < BR::KX; ++k) {
    const int u = tid + T * k;
    if (u < BR::UX) {
      int rg, pg;
      unit_of(u, rg, pg);
      const int r0 = 4 * rg;
      if constexpr (BR::XPAIR) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          quad q;
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = (E)IO::X::cvt2(r.x2[k][e], c);
          *reinterpret_cast<quad *>(&sXT[(2 * pg + c) * LDJ + r0]) = q;
        }
      } else {
        f32x4 v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = IO::X::cvt4(r.x[k][e]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          quad q;
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = (E)v[e][c];
          *reinterpret_cast<quad *>(&sXT[(4 * pg + c) * LDJ + r0]) = q;
        }
      }
    }
  }
}

// The z gate of one 64-token block, staged like x so each row's epilogue
// finds it in LDS: unit u holds row u/8, columns 8 (u%8) .. +8.
typedef unsigned int u32x4v __attribute__((vector_size(16)));
typedef unsigned int u32x2v __attribute__((vector_size(8)));
template <int T>
struct ZRaw {
  static constexpr int K = 512 / T;
  u32x4v lo[K], hi[K];  // 8 fp32, or 8 bf16 in lo
};

template <int T>
__device__ __forceinline__ void load_z(rsrc_t rz, bool bf16, uint32_t zs, uint32_t h, uint32_t tb,
                                       ZRaw<T> &r) {
#pragma unroll
  for (int k = 0; k < ZRaw<T>::K; ++k) {
    const int u = threadIdx.x + T * k;
    const uint32_t off = (tb + u / 8) * zs + h * kP + 8 * (u % 8);
    if (bf16) {
      r.lo[k] = IoBF16::load8(rz, off);
    } else {
      r.lo[k] = __builtin_amdgcn_raw_buffer_load_b128(rz, off * 4, 0, 0);
      r.hi[k] = __builtin_amdgcn_raw_buffer_load_b128(rz, off * 4 + 16, 0, 0);
    }
  }
}

template <int T>
__device__ __forceinline__ void store_z(const ZRaw<T> &r, bool bf16, float *sZ) {
  constexpr int LDZ = kP + 4;
#pragma unroll
  for (int k = 0; k < ZRaw<T>::K; ++k) {
    const int u = threadIdx.x + T * k;
    f32x4 lo, hi;
    if (bf16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = IoBF16::cvt8(r.lo[k], e);
        hi[e] = IoBF16::cvt8(r.lo[k], 4 + e);
      }
    } else {
      lo = __builtin_bit_cast(f32x4, r.lo[k]);
      hi = __builtin_bit_cast(f32x4, r.hi[k]);
    }
    // lanes 4..7 of each group of 8 write their halves in the other order,
    // so each 16-byte write instruction covers all 32 banks once
    float *dst = &sZ[(u / 8) * LDZ + 8 * (u % 8)];
    const bool sw = (u & 4) != 0;
    *reinterpret_cast<f32x4 *>(dst + (sw ? 4 : 0)) = sw ? hi : lo;
    *reinterpret_cast<f32x4 *>(dst + (sw ? 0 : 4)) = sw ? lo : hi;
  }
}

// Ownership of the P x N state by the W waves: wave w holds rows p in
// [16 (w%4), +16) and NN = N/(4W/4... ) consecutive 16-column tiles starting
// at tile (w/4) NN, in MFMA accumulator layout.
template <int N, int W>
struct StateSplit {
  static constexpr int NN = (N / 16) / (W / 4);  // n-tiles per wave
  static __device__ __forceinline__ int row(int r) {
    return 16 * ((threadIdx.x >> 6) & 3) + 4 * ((threadIdx.x & 63) >> 4) + r;
  }
  static __device__ __forceinline__ int col(int t) {
    return 16 * ((threadIdx.x >> 8) * NN + t) + (threadIdx.x & 15);
  }
};

// Main-pass waves per workgroup for a chunk size.
template <int Q> constexpr int main_waves() { return Q == 256 ? 8 : 4; }

// Group records in the workspace (aggregates, entering states) are kept in
// the main pass's register order: slice t (of NN) of main-pass thread i, the
// four rows row(0..3) of column col(t), sits at float (t * T + i) * 4 (T
// main-pass threads), so each slice of a record is one coalesced 16-byte
// load per lane.  rec_index maps the element (row p, column n) of the P x N
// state to its position; rec_element is the inverse.
template <int N, int WM>
__device__ __forceinline__ uint32_t rec_index(int row, int col) {
  constexpr int NN = StateSplit<N, WM>::NN, T = 64 * WM;
  const int tile = col >> 4;
  const int w = 4 * (tile / NN) + (row >> 4);
  const int tid = 64 * w + 16 * ((row & 15) >> 2) + (col & 15);
  return (uint32_t)(((tile % NN) * T + tid) * 4 + (row & 3));
}

template <int N, int WM>
__device__ __forceinline__ void rec_element(uint32_t e, int &row, int &col) {
  constexpr int NN = StateSplit<N, WM>::NN, T = 64 * WM;
  const int r = (int)(e & 3), t = (int)((e >> 2) / T), tid = (int)((e >> 2) % T);
  const int w = tid >> 6, lane = tid & 63;
  row = 16 * (w & 3) + 4 * (lane >> 4) + r;
  col = 16 * ((w >> 2) * NN + t) + (lane & 15);
}

// chunk_state on one staged block: S += X^T diag(w) B over the block's 64
// tokens, for this wave's share of the state.
template <int N, int MM, int W>
__device__ __forceinline__ void state_block_mma(const typename Mma<MM>::T *sXT,
                                                const typename Mma<MM>::T *sBT, f32x4 *sacc) {
  using frag = typename Mma<MM>::frag;
  constexpr int LDJ = kJB + 8;
  constexpr int NN = StateSplit<N, W>::NN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, lq = lane >> 4;
  const int ps = w & 3, n0 = (w >> 2) * NN;
#pragma unroll 1
  for (int kb = 0; kb < kJB / 32; ++kb) {
    const frag a = *reinterpret_cast<const frag *>(&sXT[(16 * ps + lr) * LDJ + 32 * kb + 8 * lq]);
#pragma unroll
    for (int t = 0; t < NN; ++t) {
      const frag bf =
          *reinterpret_cast<const frag *>(&sBT[(16 * (n0 + t) + lr) * LDJ + 32 * kb + 8 * lq]);
      sacc[t] = mma(a, bf, sacc[t]);
    }
  }
}

// Work split of a chunk's Q output rows (NT = Q/16 row tiles) over W waves.
// Row tiles are dealt in mirrored sets (s, 7-s, 8+s, 15-s, ...) so the
// causal work per SIMD is even; with fewer tiles than waves the waves
// sharing a SIMD split the head dim instead.
template <int Q, int W>
struct RowSplit {
  static constexpr int NT = Q / 16;
  static constexpr int NR = NT >= W ? NT / W : 1;   // row tiles per wave
  static constexpr int PT = NT >= W ? 4 : 4 * NT / W;  // p-tiles per wave
  static __device__ __forceinline__ int tile(int k, int w) {
    if (NT < W) return w % NT;                // NT = 4, W = 8
    if (W == 4) {                             // tiles w, 7-w, 8+w, 15-w
      const int pi = k >> 1;
      return (k & 1) ? 8 * pi + 7 - w : 8 * pi + w;
    }
    // W = 8: SIMD s = w%4 owns tiles s, 7-s (NT = 8) or s, 7-s, 8+s, 15-s
    // (NT = 16), shared by its two waves
    const int s = w & 3, hf = w >> 2;
    if (NT == 8) return hf ? 7 - s : s;
    return hf ? (k ? 8 + s : 7 - s) : (k ? 15 - s : s);
  }
  static __device__ __forceinline__ int pt0(int w) { return NT < W ? PT * (w / NT) : 0; }
};

__device__ __forceinline__ int nblocks(int Qc) { return (Qc + kJB - 1) / kJB; }

// ---------------------------------------------------------------- kernels

// First pass (only when a sequence is split into several chunk groups): the
// state each of the first ngroups-1 groups of a (b, h) builds from a zero
// start (its aggregate) and the group's total decay, for HW heads of one B/C
// group in one workgroup.  The heads share the group's B rows, so each
// 64-token block of B is loaded and staged once for all of them (transposed,
// unweighted), and each head's x block is staged with that head's
// chunk-state weights w_j = exp(Lam_end - Lam_j) delta_j folded in:
// S_h += (w_h x_h)^T B.  Four waves per head carry its state in the main
// pass's split; two blocks are in flight (a block's registers are refilled
// with the block two ahead as soon as it is staged in LDS).
//
// Tiles are ordered (b, g, group, head set) and dealt in contiguous runs to
// the XCDs (workgroup n on XCD n % 8), so the head sets that read one B block
// share an L2; packed calls deal them round-robin (rows differ in length).
__device__ __forceinline__ bool decode_state_tile(const Params &p, int hw, int64_t &b, int64_t &g,
                                                  int64_t &s, int64_t &j) {
  const int64_t sets = udiv32(p.H, p.G) / hw, ng1 = p.ngroups - 1;
  const int64_t total = p.batch * p.G * ng1 * sets;
  const int64_t n = blockIdx.x;
  const int64_t T = p.cu_seqlens ? n : (n % 8) * ((total + 7) / 8) + n / 8;
  if (T >= total) return false;
  s = umod32(T, sets);
  int64_t rest = udiv32(T, sets);
  j = umod32(rest, ng1);
  rest = udiv32(rest, ng1);
  g = umod32(rest, p.G);
  b = udiv32(rest, p.G);
  return true;
}

inline int64_t state_grid(const Params &p, int hw) {
  const int64_t total = p.batch * p.G * (p.ngroups - 1) * ((p.H / p.G) / hw);
  return p.cu_seqlens ? total : 8 * ((total + 7) / 8);
}

template <int Q, int N, int MM, class IO, int HW>
__global__ __launch_bounds__(256 * HW) void ssd_group_state_kernel(Params p) {
  constexpr int T = 256 * HW, NB = Q / kJB;
  using E = typename Mma<MM>::T;
  using quad = typename Mma<MM>::quad;
  constexpr int LDJ = kJB + 8;
  constexpr int NN = StateSplit<N, 4>::NN;
  constexpr int UB = 16 * (N / 4);              // B staging units (4 tokens x 4 columns)
  constexpr int KU = (UB + T - 1) / T;          // B units per thread
  __shared__ __attribute__((aligned(16))) E sBT[N * LDJ];
  __shared__ __attribute__((aligned(16))) E sXT[HW][kP * LDJ];
  __shared__ __attribute__((aligned(16))) ChunkLds<Q> clb[HW][2];

  int64_t b, g, s, j;
  if (!decode_state_tile(p, HW, b, g, s, j)) return;
  const RowSpan rs = row_span(p, b);
  if (j >= row_groups(p, rs.len) - 1) return;  // the row's last group, or past its end
  const int hh = (int)(threadIdx.x >> 8);       // head of the set this thread works for
  const int tid = (int)(threadIdx.x & 255);     // thread index within that head's four waves
  const int64_t hpg = udiv32(p.H, p.G);
  const int64_t h = g * hpg + s * HW + hh;
  const int64_t bh = b * p.H + h;
  const SeqView<N, IO> sv(p, rs, h, g);

  f32x4 sacc[NN];
#pragma unroll
  for (int t = 0; t < NN; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lgrp = 0.f, lend2 = 0.f;
  const int64_t c_begin = j * p.cpg;  // never the last group: all its chunks are full
  const int nblk = (int)p.cpg * NB;
  const uint32_t tg = (uint32_t)(c_begin * Q);
  auto tok = [&](int i) { return tg + (uint32_t)(kJB * (i < nblk ? i : nblk - 1)); };

  const rsrc_t rdt = make_rsrc(p.dt + rs.start * p.dts, (uint32_t)(rs.len * p.dts * 4));
  const float a_h = p.A[h], bias = p.dt_bias ? p.dt_bias[h] : 0.f;

  // one block in registers: this thread's B units and its head's x unit
  struct Raw {
    typename IO::BC::raw4 b[KU][4];
    typename IO::X::raw4 x[4];
    float dt;  // raw dt of the block one chunk later (see below)
  };
  int rgx, pgx;
  unit_of(tid, rgx, pgx);
  auto load = [&](int i, Raw &r) {
    const uint32_t tb = tok(i);
#pragma unroll
    for (int k = 0; k < KU; ++k) {
      const int u = (int)threadIdx.x + T * k;
      const bool ok = UB % T == 0 || u < UB;
      int rg, ng;
      unit_of(u, rg, ng);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r.b[k][e] = IO::BC::load4(sv.B, ok ? sv.boff(tb + 4 * rg + e, 4 * ng) : kNoElem);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) r.x[e] = IO::X::load4(sv.x, sv.xoff(tb + 4 * rgx + e, 4 * pgx));
    // the block carries the raw dt of the block at the same position one
    // chunk later (token 64 i + t of the group for block i + NB, thread t <
    // 64 of its head; later threads repeat token 63); it is staged in the
    // next chunk's LDS scalars when the block is staged, so its wait is the
    // block's own
    r.dt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        rdt, ((tg + (uint32_t)(kJB * (i + NB)) + dt_token(kJB, tid)) * sv.dts + sv.h) * 4, 0, 0));
  };
  auto store = [&](const Raw &r, int jb, const ChunkLds<Q> &cl) {
#pragma unroll
    for (int k = 0; k < KU; ++k) {
      const int u = (int)threadIdx.x + T * k;
      if (UB % T == 0 || u < UB) {
        int rg, ng;
        unit_of(u, rg, ng);
        f32x4 v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = IO::BC::cvt4(r.b[k][e]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          quad q;
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = (E)v[e][c];
          *reinterpret_cast<quad *>(&sBT[(4 * ng + c) * LDJ + 4 * rg]) = q;
        }
      }
    }
    const int r0 = 4 * rgx;
    const f32x4 wgt = *reinterpret_cast<const f32x4 *>(&cl.w[kJB * jb + r0]);
    f32x4 v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = IO::X::cvt4(r.x[e]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      quad q;
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = (E)(wgt[e] * v[e][c]);
      *reinterpret_cast<quad *>(&sXT[hh][(4 * pgx + c) * LDJ + r0]) = q;
    }
  };

  stage_dt<Q>(load_dt(rdt, sv.dts, sv.h, tg, Q, tid), clb[hh][c_begin & 1], tid);
  // (scheduling barriers keep every buffer's loads in the same issue order
  // before and inside the loop, so the compiler can count them exactly)
  Raw nx0, nx1;
  load(0, nx0);
  __builtin_amdgcn_sched_barrier(0);
  load(1, nx1);
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();

  const int lane = tid & 63, wl = tid >> 6, lr = lane & 15, lq = lane >> 4;
  auto step = [&](Raw &buf, int i) {
    const int jb = i % NB;
    const int64_t c = c_begin + i / NB;
    ChunkLds<Q> &cl = clb[hh][c & 1];
    if (jb == 0) {
      bool factored;
      chunk_prep<Q>(p, (uint32_t)(c * Q), (uint64_t)rs.len, a_h, bias, cl, lend2, factored, tid);
      const float dec = fast_exp2(lend2);
#pragma unroll
      for (int t = 0; t < NN; ++t) sacc[t] *= dec;
      lgrp += lend2;
    }
    lds_barrier();
    store(buf, jb, cl);
    // dt of the same block position in chunk c+1, into the other buffer
    // (its readers from chunk c-1 passed the barrier above)
    clb[hh][(c + 1) & 1].dts[kJB * jb + dt_token(kJB, tid)] = buf.dt;
    lds_barrier();
    load(i + 2, buf);  // past the group's end: its last block, unused
    __builtin_amdgcn_sched_barrier(0);
    // chunk_state of this block: S += (w x)^T B for this wave's share
#pragma unroll 1
    for (int kb = 0; kb < kJB / 32; ++kb) {
      using frag = typename Mma<MM>::frag;
      const frag a =
          *reinterpret_cast<const frag *>(&sXT[hh][(16 * wl + lr) * LDJ + 32 * kb + 8 * lq]);
#pragma unroll
      for (int t = 0; t < NN; ++t) {
        const frag bf =
            *reinterpret_cast<const frag *>(&sBT[(16 * t + lr) * LDJ + 32 * kb + 8 * lq]);
        sacc[t] = mma(a, bf, sacc[t]);
      }
    }
  };
  int i = 0;
  for (; i + 1 < nblk; i += 2) {
    step(nx0, i);
    step(nx1, i + 1);
  }
  if (i < nblk) step(nx0, i);
  // the aggregate, in the main pass's register order
  const int64_t slot = bh * (p.ngroups - 1) + j;
  float *dst = p.grp_state + slot * (int64_t)(kP * N);
  // (the four rows of a fragment are consecutive in the record, and
  // consecutive lanes' fragments adjacent: one coalesced 16-byte store each;
  // device scope, so the aggregates are in memory when the last workgroup
  // ends instead of dirty in the L2s: 20.6 -> 19.4 us before the headline's
  // main pass)
  constexpr int WM = main_waves<Q>();
  const rsrc_t rd = make_rsrc(dst, (uint32_t)(kP * N * 4));
#pragma unroll
  for (int t = 0; t < NN; ++t)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, sacc[t]), rd,
                                           rec_index<N, WM>(16 * wl + 4 * lq, 16 * t + lr) * 4, 0,
                                           kSc1);
  if (tid == 0) p.grp_lam[slot] = lgrp;
}

// state_passing across chunk groups as its own pass (used when sequences
// have more than kFoldGroups+1 groups; elementwise over P*N, sequential over
// groups): S = exp(Lam_grp) S + S_grp; slot j is overwritten with the state
// entering group j+1.
template <int N, int WM>
__global__ __launch_bounds__(256) void ssd_group_passing_kernel(Params p) {
  constexpr int PN = kP * N;
  constexpr int64_t blocks_per_bh = PN / 256;
  const int64_t bh = blockIdx.x / blocks_per_bh;
  const int64_t e = (blockIdx.x % blocks_per_bh) * 256 + threadIdx.x;  // record order
  float S = 0.f;
  if (p.h0) {
    int row, col;
    rec_element<N, WM>((uint32_t)e, row, col);
    S = p.h0[bh * PN + row * N + col];
  }
  const int64_t ng1 = p.ngroups - 1;
  const int64_t ng1_row = row_groups(p, row_span(p, udiv32(bh, p.H)).len) - 1;  // filled slots
  // KS slots at a time: their loads are all in flight before the chain uses
  // them (a slot index past the filled ones repeats the last, unused); the
  // entering states are stored with device scope, like the aggregates
  constexpr int KS = 8;
  auto slot_rsrc = [&](int64_t jj) { return make_rsrc(p.grp_state + (bh * ng1 + jj) * PN, PN * 4); };
  for (int64_t j0 = 0; j0 < ng1_row; j0 += KS) {
    float v[KS], lam[KS];
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      const int64_t jj = j0 + q < ng1_row ? j0 + q : ng1_row - 1;
      v[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(slot_rsrc(jj), (uint32_t)e * 4, 0, 0));
      lam[q] = p.grp_lam[bh * ng1 + jj];
    }
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      if (j0 + q >= ng1_row) break;
      S = fast_exp2(lam[q]) * S + v[q];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S), slot_rsrc(j0 + q), (uint32_t)e * 4, 0,
                                            kSc1);
    }
  }
}

// ---------------------------------------------------------------- fused norm
// The gated RMSNorm that follows the scan (page "ops-transformer MambaV2
// 算子套件", §4.6, in the chain order of its §2) normalises each token over
// groups of k heads.  Every head is a different workgroup, so the k
// workgroups of a group exchange, once per chunk, the per-token partial
// sums of squares of their 64 channels.  Each partial is one 64-bit record:
// the fp32 sum in the low half and the call's tag in the high half, stored
// with one device-scope (sc1, written through its XCD's L2) store, so a
// reader that sees the tag sees the sum.  A wave that needs its rows' sums
// loads the k members' records with device-scope loads and loads again
// until every tag is this call's.  The tag is one more than an epoch word
// that the last workgroup of every launch advances, so records left by an
// earlier call (or by an earlier replay of a captured graph) never match.
//
// The k workgroups of a group are consecutive tiles, which are consecutive
// in the dispatch order of one XCD (decode_tile), so a waiting wave's
// partners are already resident or are dispatched once earlier, complete
// groups finish (at most one group per XCD is partly dispatched, and k is
// far below the workgroups an XCD holds).  The wait is still bounded (20 ms
// of the 100 MHz real-time counter): on a time-out *error_flag is set to 2
// and those rows come out undefined, but the kernel ends.
constexpr uint64_t kNormTicks = 2000000;    // 20 ms

// Sum over the 16 lanes of a quarter-wave (lanes 16q .. 16q+15); every lane
// ends with the same value (each butterfly stage adds the same two terms).
__device__ __forceinline__ f32x4 quarter_sum(f32x4 v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1)
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] += __shfl_xor(v[r], m, 64);
  return v;
}

// This launch's tag: the epoch the previous launch left, plus one.
__device__ __forceinline__ uint32_t norm_tag(const Params &p) {
  return (uint32_t)__hip_atomic_load(p.norm_sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
}

// The end of a workgroup (every one, early exits included): the last of the
// launch zeroes the count and advances the epoch for the next launch.  Every
// workgroup has read its tag and all its records before it counts itself.
__device__ __forceinline__ void norm_done(const Params &p) {
  if (threadIdx.x != 0) return;
  const uint64_t old =
      __hip_atomic_fetch_add(p.norm_sync + 1, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old + 1 == (uint64_t)gridDim.x) {
    __hip_atomic_store(p.norm_sync + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(p.norm_sync, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The records of one member (head hm) for four consecutive rows of a chunk.
struct NormRec {
  u32x4v a, b;  // rows r, r+1 and r+2, r+3: (sum bits, tag) each
};
__device__ __forceinline__ NormRec norm_load(rsrc_t rx, int Q, int64_t hm, int row) {
  const uint32_t off = (uint32_t)((hm * Q + row) * 8);
  NormRec r;
  r.a = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, kSc1));
  r.b = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16, 0, kSc1));
  return r;
}
__device__ __forceinline__ bool norm_ready(const NormRec &r, uint32_t tag) {
  return r.a[1] == tag && r.a[3] == tag && r.b[1] == tag && r.b[3] == tag;
}
// Wait until member hm's records carry `tag` (`r` holds a first load);
// returns their four sums.
__device__ __forceinline__ f32x4 norm_take(const Params &p, rsrc_t rx, int Q, int64_t hm, int row,
                                           uint32_t tag, NormRec r) {
  if (!norm_ready(r, tag)) {
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + kNormTicks;
    for (;;) {
      __builtin_amdgcn_s_sleep(1);
      r = norm_load(rx, Q, hm, row);
      if (norm_ready(r, tag)) break;
      if (__builtin_amdgcn_s_memrealtime() > t_end) {
        if (p.error_flag)
          __hip_atomic_store(p.error_flag, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  return f32x4{__uint_as_float(r.a[0]), __uint_as_float(r.a[2]), __uint_as_float(r.b[0]),
               __uint_as_float(r.b[2])};
}

// Main pass: chunk_scan over the chunks of one group with W waves, carrying
// the state.  Per chunk: the inter-chunk term C.S_in^T from the carried
// state, then per 64-token block the intra-chunk term, the block's
// contribution to the carried state and the epilogue of the rows the block
// completes; the next block's loads are issued before its matrix work.
template <int Q, int N, int MM, class IO, int W, bool HAS_Z, bool HAS_NORM>
__global__ __launch_bounds__(64 * W, 2) void ssd_chunk_scan_kernel(Params p) {
  constexpr int T = 64 * W;
  using E = typename Mma<MM>::T;
  using frag = typename Mma<MM>::frag;
  using quad = typename Mma<MM>::quad;
  using RS = RowSplit<Q, W>;
  using SS = StateSplit<N, W>;
  constexpr int NR = RS::NR, PT = RS::PT;
  constexpr int KB = N / 32;  // K blocks over the state dim
  constexpr int NN = SS::NN;
  constexpr int LDN = N + 8, LDJ = kJB + 8, LDZ = kP + 4;
  // hoist the fp16 M.X operand fragments out of the row-tile loop only when
  // the state and output accumulators take fewer than 64 registers (with 64,
  // as for 128-token chunks of a 128-wide state, the hoisted fragments spill;
  // the fp32 check path keeps them unhoisted too)
  constexpr bool kHoistX = MM != kMmaF32 && 4 * NN + 4 * NR * PT < 64;
  __shared__ __attribute__((aligned(16))) E sB[kJB * LDN];
  __shared__ __attribute__((aligned(16))) E sBT[N * LDJ];
  __shared__ __attribute__((aligned(16))) E sXT[kP * LDJ];
  __shared__ __attribute__((aligned(16))) E sS[kP * LDN];
  __shared__ __attribute__((aligned(16))) float sZ[HAS_Z ? kJB * LDZ : 4];
  __shared__ __attribute__((aligned(16))) ChunkLds<Q> clb[2];
  __shared__ float snw[HAS_NORM ? kP : 1];

  // fused norm with an exchange: every workgroup counts itself out at its end
  const bool nx = HAS_NORM && p.norm_k > 1;
  int64_t b, h, j;
  if (!decode_tile(p, p.ngroups, b, h, j, true)) {
    if (nx) norm_done(p);
    return;
  }
  if (p.cu_seqlens && p.error_flag && j == 0 && threadIdx.x == 0 && offsets_break_contract(p, b))
    __builtin_amdgcn_raw_buffer_store_b32(1u, make_rsrc(p.error_flag, 4u), 0, 0, 0);
  const RowSpan rs = row_span(p, b);
  const int64_t ng_row = row_groups(p, rs.len), nc_row = row_chunks(p, rs.len);
  if (j >= ng_row) {  // past the end of a shorter packed sequence
    if (nx) norm_done(p);
    return;
  }
  const uint32_t ntag = nx ? norm_tag(p) : 0u;
  // the wave index is uniform: read it into a scalar so per-wave tests branch
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int pt0 = RS::pt0(w);
  const int64_t g = udiv32(h, udiv32(p.H, p.G));
  const SeqView<N, IO> sv(p, rs, h, g);
  const uint64_t lhp = (uint64_t)rs.len * p.H * kP, ohp = (uint64_t)rs.start * p.H * kP;
  const int osz = p.out_bf16 ? 2 : 4, zsz = p.z_bf16 ? 2 : 4;
  const rsrc_t rout = make_rsrc(static_cast<char *>(p.out) + ohp * osz, (uint32_t)(lhp * osz));
  const rsrc_t rz = make_rsrc(HAS_Z ? static_cast<const char *>(p.z) + rs.start * p.zs * zsz : nullptr,
                              HAS_Z ? (uint32_t)(rs.len * p.zs * zsz) : 0u);
  const bool z_bf16 = p.z_bf16 != 0;
  const float Dh = p.D ? p.D[h] : 0.f;
  // fused norm: the head's 64 channel weights, staged in LDS (read after
  // the prologue's barrier)
  if constexpr (HAS_NORM) {
    if (w == 0) snw[lane] = p.norm_w[h * kP + lane];  // (a wave-uniform branch)
  }
  const int64_t bh = b * p.H + h;
  const int64_t c_begin = j * p.cpg;
  const int64_t c_end = (c_begin + p.cpg < nc_row) ? c_begin + p.cpg : nc_row;
  auto qc_of = [&](int64_t c) { return (int)((rs.len - c * Q) < Q ? (rs.len - c * Q) : Q); };

  // prefetch registers: next 64-token block (and its z), next chunk's C rows
  // and records
  BlockRaw<N, IO, T> nxt;
  ZRaw<T> nz;
  auto load_zb = [&](uint32_t tb) {
    if (HAS_Z) load_z<T>(rz, z_bf16, (uint32_t)p.zs, sv.h, tb, nz);
  };
  const rsrc_t rdt = make_rsrc(p.dt + rs.start * p.dts, (uint32_t)(rs.len * p.dts * 4));
  const float a_h = p.A[h], bias = p.dt_bias ? p.dt_bias[h] : 0.f;
  typename IO::BC::raw8 craw[NR][KB];
  auto load_c = [&](uint32_t t0) {
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        craw[k][kb] = IO::BC::load8(sv.C, sv.boff(t0 + 16 * RS::tile(k, w) + lr, 32 * kb + 8 * lq));
  };
  // C rows are prefetched during the previous chunk's last block when they
  // fit in 16 registers, else loaded at the start of their chunk
  constexpr bool kPrefetchC = NR * KB * sizeof(typename IO::BC::raw8) <= 64;

  // Prologue.  Loads retire in issue order: the first two chunks' dt are
  // asked for first, so staging dt does not wait for the first block; the
  // block (its z, the first chunk's prefetched C rows) follows, then the
  // initial state and the first R group aggregates, which arrive with the
  // block instead of one round trip after it.
  // dt two chunks ahead in registers, one chunk ahead in LDS.
  const float dt0 = load_dt(rdt, sv.dts, sv.h, (uint32_t)(c_begin * Q), Q);
  float dtr = load_dt(rdt, sv.dts, sv.h, (uint32_t)((c_begin + 1 < c_end ? c_begin + 1 : c_begin) * Q), Q);

  // state entering this group: state_passing over the groups before it,
  // S = exp(Lam_grp[i]) S + S_grp[i] for i < j starting from h0 (or zero),
  // elementwise in this thread's share of the state; the aggregates are
  // loaded R at a time through a range holding slots i_begin..j-1 (a missing
  // h0, and slots past j-1, read as zeros through the range check).  When the
  // passing pass already chained the groups, slot j-1 holds the entering
  // state: the same loop then runs once, from zero.
  f32x4 sacc[NN];
  {
    const bool from_zero = p.chained && j > 0;
    const int64_t i_begin = from_zero ? j - 1 : 0;
    const float *h0 = (p.h0 && !from_zero) ? p.h0 + bh * (int64_t)(kP * N) : nullptr;
    const rsrc_t ri = make_rsrc(h0, h0 ? (uint32_t)(kP * N * 4) : 0u);
    constexpr int R = 16 / NN > 0 ? 16 / NN : 1;
    const int64_t ng1 = p.ngroups - 1;
    // at most kFoldGroups + 1 slots (one when chained): far below 2^32 bytes
    const rsrc_t ra = make_rsrc(j > i_begin ? p.grp_state + (bh * ng1 + i_begin) * (int64_t)(kP * N)
                                            : nullptr,
                                (uint32_t)((j - i_begin) * (kP * N * 4)));
    const float *glam = p.grp_lam + bh * ng1;
    load_block<N, IO, T>(sv, (uint32_t)(c_begin * Q), nxt);
    load_zb((uint32_t)(c_begin * Q));
    if (kPrefetchC) load_c((uint32_t)(c_begin * Q));
    f32x4 v[R][NN];
    auto load_aggs = [&](int64_t i0) {
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int t = 0; t < NN; ++t)
          v[q][t] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                         ra, (uint32_t)(((i0 - i_begin + q) * (kP * N) + (t * T + threadIdx.x) * 4) * 4),
                         0, 0));
    };
#pragma unroll
    for (int t = 0; t < NN; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sacc[t][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            ri, (uint32_t)(SS::row(r) * N + SS::col(t)) * 4, 0, 0));
    load_aggs(i_begin);
    stage_dt<Q>(dt0, clb[c_begin & 1]);
    for (int64_t i0 = i_begin; i0 < j; i0 += R) {
      if (i0 != i_begin) load_aggs(i0);
#pragma unroll
      for (int q = 0; q < R; ++q) {
        if (i0 + q >= j) break;
        const float dec = fast_exp2(glam[i0 + q]);
#pragma unroll
        for (int t = 0; t < NN; ++t) sacc[t] = dec * sacc[t] + v[q][t];
      }
    }
#pragma unroll
    for (int t = 0; t < NN; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) sS[SS::row(r) * LDN + SS::col(t)] = (E)sacc[t][r];
  }
  lds_barrier();  // the first chunk's staged dt

  // output accumulators of this wave's row tiles (with the fused norm they
  // hold the chunk's gated y until its exchange ends at the chunk's end)
  f32x4 yacc[NR][PT];
  // the epilogue's store of four rows of a tile from token `tok` of the row
  // (rows past the sequence end are dropped by the buffer range check)
  const uint32_t rstep = sv.H * kP;  // elements between consecutive tokens of out
  auto store_rows = [&](uint32_t tok, const f32x4 (&yv)[PT]) {
    const uint32_t off0 = sv.ooff(tok, 16 * pt0 + lr);
    if (p.out_bf16) {
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(yv[pt][r]), rout,
                                                (off0 + r * rstep + 16 * pt) * 2, 0, 0);
    } else {
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv[pt][r]), rout,
                                                (off0 + r * rstep + 16 * pt) * 4, 0, 0);
    }
  };
  // fused norm: chunk cc's exchange record (partial sums of squares per
  // head and token), and the end of its exchange -- the wait, then every
  // tile of the chunk (its gated y in the accumulators) normalised and
  // stored; nbc = the chunk's 64-token blocks
  auto norm_record = [&](int64_t cc) {
    return make_rsrc(nx ? p.norm_rec + ((b * p.nchk_row + cc) * p.H) * Q : nullptr,
                     nx ? (uint32_t)(p.H * Q * 8) : 0u);
  };
  const int64_t h0n = h - umod32(h, p.norm_k);  // the norm group's first head
  // the sums over the group's members for rows crow .. crow+3 of chunk cc
  // (lane lr takes members lr, lr+16; then the quarter-wave adds them up)
  auto norm_sums = [&](int64_t cc, int crow) {
    const rsrc_t rxc = norm_record(cc);
    f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int m = lr; m < p.norm_k; m += 16)
      tot += norm_take(p, rxc, Q, h0n + m, crow, ntag, norm_load(rxc, Q, h0n + m, crow));
    return quarter_sum(tot);
  };
  auto norm_scale_store = [&](int64_t cc, int crow, f32x4 tot, f32x4 (&yv)[PT]) {
    const float inv_n = 1.f / (float)(p.norm_k * kP);
    float rstd[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) rstd[r] = __builtin_amdgcn_rsqf(tot[r] * inv_n + p.norm_eps);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const float wc = snw[16 * (pt0 + pt) + lr];
#pragma unroll
      for (int r = 0; r < 4; ++r) yv[pt][r] *= rstd[r] * wc;
    }
    store_rows((uint32_t)(cc * Q + crow), yv);
  };
  auto own_sums = [&](const f32x4 (&yv)[PT]) {
    f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
      for (int r = 0; r < 4; ++r) tot[r] += yv[pt][r] * yv[pt][r];
    return quarter_sum(tot);
  };
  // every tile of chunk cc (its gated y in the accumulators) normalised and
  // stored; nbc = the chunk's 64-token blocks
  auto norm_finish = [&](int64_t cc, int nbc) {
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int row0 = 16 * RS::tile(k, w);
      if ((row0 >> 6) >= nbc) continue;  // past a ragged chunk's last block
      const int crow = row0 + 4 * lq;    // row within the chunk, + r
      const f32x4 tot = nx ? norm_sums(cc, crow) : own_sums(yacc[k]);
      norm_scale_store(cc, crow, tot, yacc[k]);
    }
  };
  // 64-token chunks (one row tile per wave) have the registers to hold a
  // chunk's gated y for a whole chunk: their exchange arrives after the next
  // chunk's first staging (when the partials' stores are long complete) and
  // ends after that chunk's products, both off the critical path
  constexpr bool kDefer = HAS_NORM && NR == 1;
  f32x4 ydef[PT];  // (unused, and dropped by the compiler, unless kDefer)
  int64_t pend_c = -1;  // chunk whose normalisation is pending (kDefer)
  const int drow = 16 * RS::tile(0, w) + 4 * lq;  // kDefer: the tile's rows in a chunk

  for (int64_t c = c_begin; c < c_end; ++c) {
    const uint32_t t0 = (uint32_t)(c * Q);
    const int Qc = qc_of(c);
    ChunkLds<Q> &cl = clb[c & 1];
    if (!kPrefetchC) load_c(t0);
    float lend2;
    bool factored;
    chunk_prep<Q, true>(p, t0, (uint64_t)rs.len, a_h, bias, cl, lend2, factored);
    lds_barrier();
    // (read into scalars: the branches on the flag stay wave-uniform)
    lend2 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cl.lend)));
    factored = __builtin_amdgcn_readfirstlane(cl.fac) != 0;
    // chunk c-1's readers of the other buffer passed the barrier above
    stage_dt<Q>(dtr, clb[(c + 1) & 1]);
    dtr = load_dt(rdt, sv.dts, sv.h, (uint32_t)((c + 2 < c_end ? c + 2 : c) * Q), Q);

    // B operand of B.C^T and A operand of C.S^T share this layout
    frag cfr[NR][KB];
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int s = 0; s < 8; ++s) cfr[k][kb][s] = (E)IO::BC::cvt8(craw[k][kb], s);

    // inter-chunk term: Y = diag(exp(Lam)) C S_in^T
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int row0 = 16 * RS::tile(k, w);
      const f32x4 lam4 = *reinterpret_cast<const f32x4 *>(&cl.lam[row0 + 4 * lq]);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const frag sf =
              *reinterpret_cast<const frag *>(&sS[(16 * (pt0 + pt) + lr) * LDN + 32 * kb + 8 * lq]);
          acc = mma(cfr[k][kb], sf, acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= fast_exp2(lam4[r]);
        yacc[k][pt] = acc;
      }
    }

    // carried state: S <- exp(Lam_end) S, then += this chunk's S_loc below
    {
      const float dec = fast_exp2(lend2);
#pragma unroll
      for (int t = 0; t < NN; ++t) sacc[t] *= dec;
    }

    // the epilogue's pieces: a tile's y + D x with x from the staged block,
    // times the z gate from the staged z; the store of four rows of a tile
    // (rows past the sequence end are dropped by the buffer range check)
    auto gated_y = [&](int k, int lrow, f32x4 (&yv)[PT]) {
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const int col = 16 * (pt0 + pt) + lr;
        const quad xq = *reinterpret_cast<const quad *>(&sXT[col * LDJ + lrow]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float y = yacc[k][pt][r] + Dh * (float)xq[r];
          if (HAS_Z) {
            const float zz = sZ[(lrow + r) * LDZ + col];
            y *= zz * __builtin_amdgcn_rcpf(1.f + __expf(-zz));
          }
          yv[pt][r] = y;
        }
      }
    };
    const rsrc_t rxn = norm_record(c);
    const int nb = nblocks(Qc);
    // the state after this chunk is read by the next chunk of the group, or
    // is the final state; after a group's last chunk it is otherwise
    // unused (the next group starts from the aggregates), so the 128-token
    // kernel skips that chunk's chunk_state products and their staging
    // (headline 55.1 -> 53.9 us, packed 70.2 -> 69.0 us; elsewhere the
    // branches cost more than they save: gated 3.8%, H256 0.4% slower)
    constexpr bool kSkipTail = Q == 128;
    const bool keep_state = !kSkipTail || c + 1 < c_end || (p.ret_final && j == ng_row - 1);
    for (int jb = 0; jb < nb; ++jb) {
      lds_barrier();
      store_block<N, MM, IO, T, true>(nxt, jb, cl.w, sB, sBT, sXT, keep_state);
      if (HAS_Z) store_z<T>(nz, z_bf16, sZ);
      const bool def_now = kDefer && jb == 0 && pend_c >= 0;  // the pending chunk's turn
      lds_barrier();
      {
        // next block: the chunk's next one, else the next chunk's first, else
        // (last block of the group) this one again, unused
        const bool last = jb + 1 == nb;
        const uint32_t tn = !last ? t0 + kJB * (jb + 1) : (c + 1 < c_end) ? t0 + Q : t0 + kJB * jb;
        load_block<N, IO, T>(sv, tn, nxt);
        load_zb(tn);
        if (kPrefetchC && last) load_c((c + 1 < c_end) ? t0 + Q : t0);
      }
      // intra-chunk term for this wave's row tiles against tokens of block jb,
      // one 32-token sub-block at a time (its B fragments serve every row
      // tile of the wave that reaches it)
#pragma unroll 1
      for (int js = 0; js < kJB / 32; ++js) {
        const int jbase = kJB * jb + 32 * js;
        bool any = false;
#pragma unroll
        for (int k = 0; k < NR; ++k) any |= jbase <= 16 * RS::tile(k, w) + 15;
        if (!any) continue;
        frag a0[KB], a1[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          a0[kb] = *reinterpret_cast<const frag *>(&sB[(32 * js + lr) * LDN + 32 * kb + 8 * lq]);
          a1[kb] = *reinterpret_cast<const frag *>(&sB[(32 * js + 16 + lr) * LDN + 32 * kb + 8 * lq]);
        }
        // x^T fragments of the sub-block (B operand of M.X; K slots j =
        // 32 js + 4 lq + s and + 16).  When the accumulators leave room they
        // are read once for all of the wave's row tiles, ahead of the B.C^T
        // products; otherwise each row tile reads them as it needs them.
        auto x_frag = [&](int pt) {
          const E *xrow = &sXT[(16 * (pt0 + pt) + lr) * LDJ + 32 * js + 4 * lq];
          const quad lo = *reinterpret_cast<const quad *>(xrow);
          const quad hi = *reinterpret_cast<const quad *>(xrow + 16);
          frag f;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            f[s] = lo[s];
            f[4 + s] = hi[s];
          }
          return f;
        };
        frag xb[kHoistX ? PT : 1];
        if constexpr (kHoistX) {
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) xb[pt] = x_frag(pt);
        }
        const int ja0 = jbase + 4 * lq;
        const float lmid = cl.mid[jbase >> 5];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const int row0 = 16 * RS::tile(k, w);
          if (jbase > row0 + 15) continue;
          const int i = row0 + lr;
          const float li = cl.lam[i];
          // G^T[j][i] = B_j . C_i for j in [jbase, jbase+32), two 16x16 tiles
          f32x4 g0 = f32x4{0.f, 0.f, 0.f, 0.f}, g1 = g0;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            g0 = mma(a0[kb], cfr[k][kb], g0);
            g1 = mma(a1[kb], cfr[k][kb], g1);
          }
          // M[i][j] = G[i][j] exp(Lam_i - Lam_j) delta_j (j <= i), held as the
          // A operand of M.X: lane keeps row i, K slots j = jbase+4lq+r and
          // jbase+16+4lq+r.  The decay factors as exp(Lam_i - Lam_m) times
          // exp(Lam_m - Lam_j) delta_j with m the sub-block's reference token.
          float ma[4], mc[4];
          if (factored) {
            const float vi = fast_exp2(li - lmid);
            const f32x4 ua = *reinterpret_cast<const f32x4 *>(&cl.u[ja0]);
            const f32x4 uc = *reinterpret_cast<const f32x4 *>(&cl.u[ja0 + 16]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              ma[r] = g0[r] * ua[r] * vi;
              mc[r] = g1[r] * uc[r] * vi;
            }
          } else {
            const f32x4 la = *reinterpret_cast<const f32x4 *>(&cl.lam[ja0]);
            const f32x4 lc = *reinterpret_cast<const f32x4 *>(&cl.lam[ja0 + 16]);
            const f32x4 da = *reinterpret_cast<const f32x4 *>(&cl.delta[ja0]);
            const f32x4 dc = *reinterpret_cast<const f32x4 *>(&cl.delta[ja0 + 16]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              ma[r] = g0[r] * (fast_exp2(li - la[r]) * da[r]);
              mc[r] = g1[r] * (fast_exp2(li - lc[r]) * dc[r]);
            }
          }
          frag mf;
          // bf16 operands: masked in fp32, then rounded two at a time
          // (v_cvt_pk_bf16_f32; 1% on the gated workload); the fp16 form
          // below measured faster as the compiler schedules it
          if constexpr (MM == kMmaBF16) {
            if (jbase + 31 > row0) {  // the sub-block meets the diagonal: mask j > i
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                ma[r] = ja0 + r <= i ? ma[r] : 0.f;
                mc[r] = ja0 + 16 + r <= i ? mc[r] : 0.f;
              }
            }
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const Pair2<E> pa = cvt2<E>(ma[r], ma[r + 1]), pc = cvt2<E>(mc[r], mc[r + 1]);
              mf[r] = pa.x;
              mf[r + 1] = pa.y;
              mf[4 + r] = pc.x;
              mf[4 + r + 1] = pc.y;
            }
          } else if (jbase + 31 > row0) {  // the sub-block meets the diagonal: mask j > i
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              mf[r] = (E)(ja0 + r <= i ? ma[r] : 0.f);
              mf[4 + r] = (E)(ja0 + 16 + r <= i ? mc[r] : 0.f);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              mf[r] = (E)ma[r];
              mf[4 + r] = (E)mc[r];
            }
          }
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) {
            if constexpr (kHoistX) yacc[k][pt] = mma(mf, xb[pt], yacc[k][pt]);
            else yacc[k][pt] = mma(mf, x_frag(pt), yacc[k][pt]);
          }
        }
      }

      // chunk_state contribution of this block to the carried state
      if (keep_state) state_block_mma<N, MM, W>(sXT, sBT, sacc);


      // epilogue of the row tiles that lie in this block (their sums are
      // complete): + D x with x from the staged block, the z gate from the
      // staged z, store (rows past the sequence end are dropped by the buffer
      // range check)
      if constexpr (!HAS_NORM) {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const int row0 = 16 * RS::tile(k, w);
          if ((row0 >> 6) != jb) continue;
          const int lrow = row0 - kJB * jb + 4 * lq;  // row within the block, + r
          f32x4 yv[PT];
          gated_y(k, lrow, yv);
          store_rows(t0 + kJB * jb + lrow, yv);
        }
      } else {
        // fused gated RMSNorm: the gated y of the tile this wave completes
        // in this block (the row splits give a wave at most one per block)
        // replaces its accumulator until the chunk's exchange; its per-row
        // sums of squares over the head's 64 channels (this lane's PT
        // columns, then the 16 lanes that hold the same four rows) go to
        // the chunk's exchange record
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const int row0 = 16 * RS::tile(k, w);
          if ((row0 >> 6) != jb) continue;
          const int lrow = row0 - kJB * jb + 4 * lq;
          gated_y(k, lrow, yacc[k]);
          if (nx) {
            // lane r < 4 of each quarter-wave stores row r's record
            const f32x4 ss = own_sums(yacc[k]);
            if (lr < 4) {
              const float v = lr == 0 ? ss[0] : lr == 1 ? ss[1] : lr == 2 ? ss[2] : ss[3];
              const u32x2v rec = {__float_as_uint(v), ntag};
              __builtin_amdgcn_raw_buffer_store_b64(
                  __builtin_bit_cast(u32x2v, rec), rxn,
                  (uint32_t)((h * Q + row0 + 4 * lq + lr) * 8), 0, kSc1);
            }
          }
        }
        if constexpr (kDefer) {
          if (def_now) {
            const f32x4 tot = nx ? norm_sums(pend_c, drow) : own_sums(ydef);
            norm_scale_store(pend_c, drow, tot, ydef);
          }
        }
      }
    }

    if constexpr (kDefer) {
      // this chunk's gated y waits in ydef for its exchange
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) ydef[pt] = yacc[0][pt];
      pend_c = c;
    } else if constexpr (HAS_NORM) {
      norm_finish(c, nb);  // the chunk's exchange ends here
    }

    // the state entering the next chunk, as the C.S^T operand (all waves
    // finished reading sS before the block loop's barriers)
    if (!kSkipTail || c + 1 < c_end) {
#pragma unroll
      for (int t = 0; t < NN; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[SS::row(r) * LDN + SS::col(t)] = (E)sacc[t][r];
    }
  }

  if constexpr (kDefer) {
    if (pend_c >= 0) {
      const f32x4 tot = nx ? norm_sums(pend_c, drow) : own_sums(ydef);
      norm_scale_store(pend_c, drow, tot, ydef);
    }
  }

  if (p.ret_final && j == ng_row - 1) {
    float *dst = p.final_state + bh * (int64_t)(kP * N);
#pragma unroll
    for (int t = 0; t < NN; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[SS::row(r) * N + SS::col(t)] = sacc[t][r];
  }
  if (nx) norm_done(p);
}


// ---------------------------------------------------------------- launches

// The main pass chains up to this many group aggregates itself; with more
// groups a separate passing pass chains them once (measured: 8 aggregates
// per workgroup cost less than the extra pass, 15 cost more).
constexpr int64_t kFoldGroups = 8;

// Workspace (only when a sequence is cut into several chunk groups): the
// group states and group decays.
struct Plan {
  int64_t nc, cpg, ngroups;
  size_t sync_bytes;       // fused norm: epoch, finish count and the tagged partial sums
  size_t state_bytes, lam_bytes;
  // everything after the norm's part, which ssd_fwd_noalloc keeps apart
  size_t data_bytes() const { return state_bytes + lam_bytes; }
  size_t total() const { return sync_bytes + data_bytes(); }
};



// Workgroups covering `ngroups_here` chunk groups of every (b, h), as
// decode_tile deals them.
inline int64_t tile_grid(const Params &p, int64_t ngroups_here, bool late_first = false) {
  const int64_t hpg = p.H / p.G;
  if (p.cu_seqlens) {
    const int64_t units = p.batch * p.G * ngroups_here;
    return 8 * hpg * ((units + 7) / 8);
  }
  const int64_t total = p.batch * p.H * ngroups_here;
  if (late_first && ngroups_here % 2 == 0 && !p.chained) return 16 * ((total / 2 + 7) / 8);
  return 8 * ((total + 7) / 8);
}

template <int Q, int N, int MM, class IO>
ssd_status launch_all(const Params &prm, const Plan &pl, hipStream_t stream, const ssd_desc *d) {
  const int64_t bh = prm.batch * prm.H;
  const int64_t g2 = tile_grid(prm, pl.ngroups, true);  // the largest grid, checked before any launch
  if (g2 > (int64_t)UINT32_MAX) return SSD_ERR_UNSUPPORTED;
  if (pl.ngroups > 1) {
    // two heads of a B/C group per workgroup when the group has an even
    // number of heads (they share the loads and staging of B), else one
    if ((prm.H / prm.G) % 2 == 0)
      hipLaunchKernelGGL((ssd_group_state_kernel<Q, N, MM, IO, 2>),
                         dim3((unsigned)state_grid(prm, 2)), dim3(512), 0, stream, prm);
    else
      hipLaunchKernelGGL((ssd_group_state_kernel<Q, N, MM, IO, 1>),
                         dim3((unsigned)state_grid(prm, 1)), dim3(256), 0, stream, prm);
    if (prm.chained)
      hipLaunchKernelGGL((ssd_group_passing_kernel<N, main_waves<Q>()>),
                         dim3((unsigned)(bh * (kP * N / 256))), dim3(256), 0, stream, prm);
  }
  if (d->ev_main_begin && hipEventRecord(static_cast<hipEvent_t>(d->ev_main_begin), stream) != hipSuccess)
    return SSD_ERR_LAUNCH;
  // 4-wave workgroups (two per CU) for chunks of 64 and 128 tokens; 8 waves
  // for 256-token chunks, whose row tiles would not fit 4 waves' registers
  constexpr int W = main_waves<Q>();
  const dim3 grid((unsigned)g2), block(64 * W);
  if (prm.norm_w) {
    if (prm.z)
      hipLaunchKernelGGL((ssd_chunk_scan_kernel<Q, N, MM, IO, W, true, true>), grid, block, 0,
                         stream, prm);
    else
      hipLaunchKernelGGL((ssd_chunk_scan_kernel<Q, N, MM, IO, W, false, true>), grid, block, 0,
                         stream, prm);
  } else if (prm.z) {
    hipLaunchKernelGGL((ssd_chunk_scan_kernel<Q, N, MM, IO, W, true, false>), grid, block, 0,
                       stream, prm);
  } else {
    hipLaunchKernelGGL((ssd_chunk_scan_kernel<Q, N, MM, IO, W, false, false>), grid, block, 0,
                       stream, prm);
  }
  if (hipGetLastError() != hipSuccess) return SSD_ERR_LAUNCH;
  if (d->ev_main_end && hipEventRecord(static_cast<hipEvent_t>(d->ev_main_end), stream) != hipSuccess)
    return SSD_ERR_LAUNCH;
  return SSD_OK;
}

template <int Q, int N, int MM>
ssd_status dispatch_io(const Params &prm, const Plan &pl, hipStream_t s, const ssd_desc *d) {
  const bool xb = d->x_dtype == SSD_BF16, bb = d->bc_dtype == SSD_BF16;
  if (xb && bb) return launch_all<Q, N, MM, IoPair<IoBF16, IoBF16>>(prm, pl, s, d);
  if (xb) return launch_all<Q, N, MM, IoPair<IoBF16, IoF32>>(prm, pl, s, d);
  if (bb) return launch_all<Q, N, MM, IoPair<IoF32, IoBF16>>(prm, pl, s, d);
  return launch_all<Q, N, MM, IoPair<IoF32, IoF32>>(prm, pl, s, d);
}

template <int Q, int N>
ssd_status dispatch_mma(const Params &prm, const Plan &pl, hipStream_t s, const ssd_desc *d) {
  if (d->mma == SSD_MMA_F32) return dispatch_io<Q, N, kMmaF32>(prm, pl, s, d);
  if (d->mma == SSD_MMA_BF16) return dispatch_io<Q, N, kMmaBF16>(prm, pl, s, d);
  return dispatch_io<Q, N, kMmaF16>(prm, pl, s, d);
}

template <int Q>
ssd_status dispatch_n(const Params &prm, const Plan &pl, hipStream_t s, const ssd_desc *d) {
  if (d->dstate == 64) return dispatch_mma<Q, 64>(prm, pl, s, d);
  return dispatch_mma<Q, 128>(prm, pl, s, d);
}

// One chunk size's launches, each in its own translation unit.
ssd_status launch_q64(const Params &prm, const Plan &pl, hipStream_t s, const ssd_desc *d);
ssd_status launch_q128(const Params &prm, const Plan &pl, hipStream_t s, const ssd_desc *d);
ssd_status launch_q256(const Params &prm, const Plan &pl, hipStream_t s, const ssd_desc *d);

}  // namespace ssd_fwd_impl
