// Gated grouped RMSNorm for MI355X (gfx950): the operator that closes the
// chunked SSD chain, page "ops-transformer MambaV2 算子套件", section 4.6
// (mamba2_rmsnormgated): g = x * SiLU(z), then per group of dim/ngroups
// contiguous elements out = g / sqrt(mean(g^2) + eps) * w.
//
// Pure streaming work (12 bytes of HBM traffic per element, a handful of
// flops), so the design is about moving bytes: one wave64 per (row, group),
// 16-byte coalesced loads of x and z kept in registers, a DPP wavefront sum
// for the mean of squares, and one 16-byte store per loaded slot.  Group
// tails are handled by the buffer range check (loads past the group read
// zeros, stores past it are dropped).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "../../include/ssd_mi355x.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// x, z and out are touched once: their accesses carry the non-temporal
// hint (cache-policy bit nt), which measured 5-15% faster than the default
// policy; w, re-read by every row, keeps the default.
constexpr int kStream = 2;

template <int POLICY = 0>
__device__ __forceinline__ f32x4 load4(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, POLICY));
}

// Sum over the 64 lanes of a wave (DPP: shifts 1, 2, 4, 8 within rows of
// 16 lanes, then row totals broadcast to later rows); lane 63 holds the sum.
__device__ __forceinline__ float wave_sum(float v) {
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
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// K 16-byte slots per lane: groups of up to 256*K elements.  Block b covers
// group b % G of rows 4*(b / G) .. +3, one wave per row, so consecutive
// blocks stream consecutive groups of the same rows (measured 10-25% faster
// than walking the rows of one group first).  Every address is wave-uniform
// and lives in scalar registers.
template <int K, bool HAS_Z>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const float *x, const float *z,
                                                            const float *w, float *out,
                                                            int64_t rows, int gsz, int ngroups,
                                                            float eps) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t rblk = blockIdx.x / (uint32_t)ngroups;
  const int grp = (int)(blockIdx.x - rblk * (uint32_t)ngroups);
  const int64_t row = (int64_t)rblk * 4 + wave;
  if (row >= rows) return;  // the whole wave
  const int64_t base = row * ((int64_t)gsz * ngroups) + (int64_t)grp * gsz;
  const uint32_t bytes = (uint32_t)gsz * 4u;
  const rsrc_t rx = make_rsrc(x + base, bytes);
  const rsrc_t rz = make_rsrc(HAS_Z ? z + base : nullptr, HAS_Z ? bytes : 0u);
  const rsrc_t rw = make_rsrc(w + (int64_t)grp * gsz, bytes);
  const rsrc_t ro = make_rsrc(out + base, bytes);

  // All loads are issued before the first use, so a wave has 2K (3K with
  // the weight) 16-byte requests in flight; small groups also fetch w early,
  // large ones fetch it after the gate so it can reuse z's registers.
  constexpr bool kEarlyW = K <= 4;
  f32x4 g[K], zv[K], wv[K];
#pragma unroll
  for (int k = 0; k < K; ++k) g[k] = load4<kStream>(rx, (uint32_t)(lane + 64 * k) * 16u);
  if (HAS_Z) {
#pragma unroll
    for (int k = 0; k < K; ++k) zv[k] = load4<kStream>(rz, (uint32_t)(lane + 64 * k) * 16u);
  }
  if (kEarlyW) {
#pragma unroll
    for (int k = 0; k < K; ++k) wv[k] = load4(rw, (uint32_t)(lane + 64 * k) * 16u);
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (HAS_Z) {
#pragma unroll
      for (int e = 0; e < 4; ++e)  // silu(z) = z / (1 + e^-z), hardware exp2 and reciprocal
        g[k][e] *= zv[k][e] * __builtin_amdgcn_rcpf(1.f + __expf(-zv[k][e]));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += g[k][e] * g[k][e];
  }
  if (!kEarlyW) {
#pragma unroll
    for (int k = 0; k < K; ++k) wv[k] = load4(rw, (uint32_t)(lane + 64 * k) * 16u);
  }
  const float scale = 1.f / sqrtf(wave_sum(ss) / (float)gsz + eps);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const f32x4 o = g[k] * scale * wv[k];
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), ro,
                                           (uint32_t)(lane + 64 * k) * 16u, 0, kStream);
  }
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

template <int K>
ssd_status launch(const float *x, const float *z, const float *w, float *out, int64_t rows,
                  int gsz, int ngroups, float eps, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4 * ngroups)), block(256);
  if (z)
    hipLaunchKernelGGL((gated_rmsnorm_kernel<K, true>), grid, block, 0, s, x, z, w, out, rows,
                       gsz, ngroups, eps);
  else
    hipLaunchKernelGGL((gated_rmsnorm_kernel<K, false>), grid, block, 0, s, x, z, w, out, rows,
                       gsz, ngroups, eps);
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_LAUNCH;
}

}  // namespace

extern "C" ssd_status ssd_rmsnorm_gated(const float *x, const float *z, const float *w,
                                        int64_t rows, int64_t dim, int64_t ngroups, float eps,
                                        float *out, void *stream) {
  if (!x || !w || !out) return SSD_ERR_INVALID_ARG;
  if (rows < 1 || dim < 1 || ngroups < 1 || dim % ngroups != 0) return SSD_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || isinf(eps)) return SSD_ERR_INVALID_ARG;  // also rejects NaN
  if (!aligned16(x) || !aligned16(w) || !aligned16(out) || (z && !aligned16(z)))
    return SSD_ERR_INVALID_ARG;
  const int64_t gsz = dim / ngroups;
  if (gsz % 4 != 0 || gsz > 4096) return SSD_ERR_UNSUPPORTED;
  if (rows > ((int64_t)1 << 40) / dim || (rows + 3) / 4 * ngroups >= ((int64_t)1 << 31))
    return SSD_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int g = (int)gsz, G = (int)ngroups;
  if (gsz <= 256) return launch<1>(x, z, w, out, rows, g, G, eps, s);
  if (gsz <= 512) return launch<2>(x, z, w, out, rows, g, G, eps, s);
  if (gsz <= 1024) return launch<4>(x, z, w, out, rows, g, G, eps, s);
  if (gsz <= 2048) return launch<8>(x, z, w, out, rows, g, G, eps, s);
  return launch<16>(x, z, w, out, rows, g, G, eps, s);
}
