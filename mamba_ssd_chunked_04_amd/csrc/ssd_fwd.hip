// Mamba-2 SSD chunked forward for MI355X (gfx950, CDNA4): the C ABI declared in
// include/ssd_mi355x.h (validation, the plan, the workspace and the static
// scratch of ssd_fwd_noalloc); the kernels are in ssd_fwd_impl.h.
#include <mutex>

#include "ssd_fwd_impl.h"

namespace ssd_fwd_impl {

// ---------------------------------------------------------------- host side

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool is_supported_chunk(int64_t q) { return q == 64 || q == 128 || q == 256; }

// Validation of everything but pointers.
ssd_status check_shape(const ssd_desc *d, int64_t chunk) {
  if (!d) return SSD_ERR_INVALID_ARG;
  if (d->batch < 1 || d->seqlen < 1 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
      d->ngroups < 1 || chunk < 1)
    return SSD_ERR_INVALID_ARG;
  if (d->nheads % d->ngroups != 0) return SSD_ERR_INVALID_ARG;
  if (d->x_dtype != SSD_F32 && d->x_dtype != SSD_BF16 && d->x_dtype != SSD_F16)
    return SSD_ERR_INVALID_ARG;
  if (d->bc_dtype != SSD_F32 && d->bc_dtype != SSD_BF16 && d->bc_dtype != SSD_F16)
    return SSD_ERR_INVALID_ARG;
  if (d->z_dtype != SSD_F32 && d->z_dtype != SSD_BF16 && d->z_dtype != SSD_F16)
    return SSD_ERR_INVALID_ARG;
  if (d->out_dtype != SSD_F32 && d->out_dtype != SSD_BF16 && d->out_dtype != SSD_F16)
    return SSD_ERR_INVALID_ARG;
  if (d->mma != SSD_MMA_F16 && d->mma != SSD_MMA_BF16 && d->mma != SSD_MMA_F32)
    return SSD_ERR_INVALID_ARG;
  if (d->chunks_per_wg < 0 || d->packed_tokens < 0) return SSD_ERR_INVALID_ARG;
  if (!(d->dt_min <= d->dt_max)) return SSD_ERR_INVALID_ARG;  // also rejects NaN
  if (d->x_dtype == SSD_F16 || d->bc_dtype == SSD_F16 || d->z_dtype == SSD_F16 ||
      d->out_dtype == SSD_F16)
    return SSD_ERR_UNSUPPORTED;
  // token strides: 0 (dense) or at least the dense row, 16-byte multiples
  const int64_t xe = d->x_dtype == SSD_BF16 ? 2 : 4, be = d->bc_dtype == SSD_BF16 ? 2 : 4;
  const int64_t ze = d->z_dtype == SSD_BF16 ? 2 : 4;
  if (d->x_stride < 0 || d->bc_stride < 0 || d->z_stride < 0 || d->dt_stride < 0)
    return SSD_ERR_INVALID_ARG;
  if ((d->x_stride && (d->x_stride < d->nheads * d->headdim || (d->x_stride * xe) % 16)) ||
      (d->bc_stride && (d->bc_stride < d->ngroups * d->dstate || (d->bc_stride * be) % 16)) ||
      (d->z_stride && (d->z_stride < d->nheads * d->headdim || (d->z_stride * ze) % 16)) ||
      (d->dt_stride && d->dt_stride < d->nheads))
    return SSD_ERR_INVALID_ARG;
  if (d->headdim != kP) return SSD_ERR_UNSUPPORTED;
  if (d->dstate != 64 && d->dstate != 128) return SSD_ERR_UNSUPPORTED;
  if (!is_supported_chunk(chunk)) return SSD_ERR_UNSUPPORTED;
  // 32-bit grid; each batch row's x/z/out and B/C slices are addressed with
  // 32-bit byte offsets
  if (d->batch > (1 << 20) || d->nheads > (1 << 20) || d->seqlen > ((int64_t)1 << 31))
    return SSD_ERR_UNSUPPORTED;
  const int64_t row_limit = (int64_t)1 << 31;
  const int64_t xs = d->x_stride ? d->x_stride : d->nheads * d->headdim;
  const int64_t bs = d->bc_stride ? d->bc_stride : d->ngroups * d->dstate;
  const int64_t zs = d->z_stride ? d->z_stride : d->nheads * d->headdim;
  const int64_t dts = d->dt_stride ? d->dt_stride : d->nheads;
  if (d->seqlen * d->nheads * d->headdim * 4 >= row_limit || d->seqlen * xs * 4 >= row_limit ||
      d->seqlen * bs * 4 >= row_limit || d->seqlen * zs * 4 >= row_limit ||
      d->seqlen * dts * 4 >= row_limit)
    return SSD_ERR_UNSUPPORTED;
  if (d->norm_weight) {
    // fused norm: groups of k = H / norm_groups heads, whose workgroups must
    // all be resident at once (k well below the workgroups of one XCD)
    if (d->norm_groups < 1 || d->nheads % d->norm_groups != 0) return SSD_ERR_INVALID_ARG;
    if (!(d->norm_eps > 0.f) || !(d->norm_eps < INFINITY)) return SSD_ERR_INVALID_ARG;
    const int64_t k = d->nheads / d->norm_groups;
    if (k > (chunk == 256 ? 16 : 32)) return SSD_ERR_UNSUPPORTED;
    // one chunk's exchange record is addressed with 32-bit byte offsets
    if (d->nheads * chunk * 4 >= row_limit) return SSD_ERR_UNSUPPORTED;
  }
  return SSD_OK;
}

// Workgroups the plan aims for on a 256-CU MI355X: one per CU for 8-wave
// workgroups (256-token chunks), two per CU for 4-wave ones.  A sequence is
// cut into chunk groups only when (b, h) pairs alone fall short of that.
int64_t target_workgroups(int64_t chunk) { return chunk == 256 ? 256 : 512; }

Plan make_plan(const ssd_desc *d, int64_t chunk) {
  Plan pl;
  pl.nc = (d->seqlen + chunk - 1) / chunk;
  const int64_t bh = d->batch * d->nheads;
  const int64_t target = target_workgroups(chunk);
  int64_t cpg;
  if (d->chunks_per_wg > 0) {
    cpg = d->chunks_per_wg;
  } else if (d->cu_seqlens) {
    // packed sequences: cut every sequence into groups of about the chunks
    // per workgroup slot that the whole call needs (counting half a ragged
    // chunk per sequence), so a long sequence among short ones does not walk
    // all its chunks in one workgroup
    const int64_t T = d->packed_tokens > 0 ? d->packed_tokens : d->batch * d->seqlen;
    const int64_t chunks = (T + chunk - 1) / chunk + d->batch / 2;
    cpg = chunks * d->nheads / target;
  } else if (bh >= target) {
    cpg = pl.nc;
  } else {
    const int64_t want = (2 * 256 + bh - 1) / bh;  // groups per (b, h)
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
  pl.sync_bytes = 0;
  if (d->norm_weight && d->nheads / d->norm_groups > 1) {
    // the epoch and the count of finished workgroups, then one 64-bit
    // record (partial sum, tag) per head and token of every chunk
    pl.sync_bytes =
        kAlign + align_up((size_t)(d->batch * pl.nc * d->nheads * chunk) * sizeof(uint64_t));
  }
  return pl;
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }
// The forward with its workspace given explicitly (the caller's buffer, or
// the static scratch of ssd_fwd_noalloc); `d->workspace` is not read here.
ssd_status fwd_impl(const void *x, const float *dt, const float *A, const void *B, const void *C,
                    const float *D, int64_t chunk, int dt_softplus, int return_final_state,
                    void *out, float *final_state, void *stream, const ssd_desc *d, void *ws,
                    size_t ws_bytes, void *sync) {
  const ssd_status st = check_shape(d, chunk);
  if (st != SSD_OK) return st;
  if (!x || !dt || !A || !B || !C || !out) return SSD_ERR_INVALID_ARG;
  if (return_final_state && !final_state) return SSD_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(out) ||
      (d->z && !aligned16(d->z)) || ((uintptr_t)dt & 3u) != 0 ||
      (d->initial_state && !aligned16(d->initial_state)) ||
      (return_final_state && !aligned16(final_state)) ||
      ((uintptr_t)d->cu_seqlens & 3u) != 0 || ((uintptr_t)d->error_flag & 3u) != 0)
    return SSD_ERR_INVALID_ARG;
  if (d->norm_weight && ((uintptr_t)d->norm_weight & 3u) != 0) return SSD_ERR_INVALID_ARG;
  const Plan pl = make_plan(d, chunk);
  // the counters sit at `sync` (the workspace's start, or the noalloc
  // scratch's own region) and everything else at `ws`
  const size_t need = sync == ws ? pl.total() : pl.data_bytes();
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return SSD_ERR_WORKSPACE;
  if (pl.sync_bytes && (!sync || ((uintptr_t)sync & 15u) != 0)) return SSD_ERR_WORKSPACE;

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
  char *wsc = static_cast<char *>(ws) + (sync == ws ? pl.sync_bytes : 0);
  prm.norm_sync = pl.sync_bytes ? static_cast<uint64_t *>(sync) : nullptr;
  prm.norm_rec = pl.sync_bytes ? reinterpret_cast<uint64_t *>(static_cast<char *>(sync) + kAlign)
                               : nullptr;
  prm.grp_state = pl.state_bytes ? reinterpret_cast<float *>(wsc) : nullptr;
  prm.grp_lam = pl.lam_bytes ? reinterpret_cast<float *>(wsc + pl.state_bytes) : nullptr;
  prm.norm_w = d->norm_weight;
  prm.norm_eps = d->norm_eps;
  prm.norm_k = d->norm_weight ? (int)(d->nheads / d->norm_groups) : 1;
  prm.nchk_row = pl.nc;
  prm.cu_seqlens = d->cu_seqlens;
  prm.error_flag = (d->cu_seqlens || d->norm_weight) ? d->error_flag : nullptr;
  prm.packed_tokens = d->cu_seqlens ? d->packed_tokens : 0;
  prm.xs = d->x_stride ? d->x_stride : d->nheads * d->headdim;
  prm.bs = d->bc_stride ? d->bc_stride : d->ngroups * d->dstate;
  prm.zs = d->z_stride ? d->z_stride : d->nheads * d->headdim;
  prm.dts = d->dt_stride ? d->dt_stride : d->nheads;
  prm.batch = d->batch;
  prm.L = d->seqlen;
  prm.Q = (int)chunk;
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
  prm.chained = pl.ngroups - 1 > kFoldGroups;

  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (chunk) {
    case 64: return launch_q64(prm, pl, s, d);
    case 128: return launch_q128(prm, pl, s, d);
    default: return launch_q256(prm, pl, s, d);
  }
}

// Scratch of ssd_fwd_noalloc: the group states and decays that ssd_fwd keeps
// in the caller's workspace, in a file-scope device array instead (every GPU
// the library runs on holds its own copy until the process ends).  In host
// code `scratch` only names the symbol; its device address on each GPU comes
// from hipGetSymbolAddress, taken once per device and kept in scratch_ptr.
constexpr size_t kScratchBytes = SSD_FWD_NOALLOC_MAX_SCRATCH;
constexpr size_t kSyncBytes = SSD_FWD_NOALLOC_SYNC_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void *ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot scratch_slots[kMaxDevices];

// Device address of `scratch` on `dev` (which must be the current device),
// or NULL if the runtime cannot give it.
void *scratch_ptr(int dev) {
  ScratchSlot &s = scratch_slots[dev];
  std::call_once(s.once, [&s] {
    s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch));
    if (s.err != hipSuccess) s.ptr = nullptr;
  });
  return s.ptr;
}

}  // namespace ssd_fwd_impl

using namespace ssd_fwd_impl;

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
  d->bc_dtype = SSD_F32;
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
  *bytes = pl.total();
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
  if (!d) return SSD_ERR_INVALID_ARG;
  return fwd_impl(x, dt, A, B, C, D, chunk, dt_softplus, return_final_state, out, final_state,
                  stream, d, d->workspace, d->workspace_bytes, d->workspace);
}

ssd_status ssd_fwd_noalloc(const void *x, const float *dt, const float *A, const void *B,
                           const void *C, const float *D, int64_t chunk, int dt_softplus,
                           int return_final_state, void *out, float *final_state, void *stream,
                           const ssd_desc *d) {
  // everything that needs no device first, so a refused call touches no GPU
  const ssd_status st = check_shape(d, chunk);
  if (st != SSD_OK) return st;
  const Plan pl = make_plan(d, chunk);
  if (pl.sync_bytes > kSyncBytes || pl.data_bytes() > kScratchBytes - kSyncBytes)
    return SSD_ERR_WORKSPACE;
  if (!x || !dt || !A || !B || !C || !out) return SSD_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERR_LAUNCH;
  hipDevice_t sdev = -1;
  if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
    return SSD_ERR_INVALID_ARG;
  if ((int)sdev != dev) return SSD_ERR_INVALID_ARG;  // the scratch address is per device
  char *base = pl.total() > 0 ? static_cast<char *>(scratch_ptr(dev)) : nullptr;
  if (pl.total() > 0 && !base) return SSD_ERR_LAUNCH;
  // the first kSyncBytes hold the fused norm's exchange (zero at load, then
  // only its epoch and tagged records), the rest the plan's other parts
  return fwd_impl(x, dt, A, B, C, D, chunk, dt_softplus, return_final_state, out, final_state,
                  stream, d, base ? base + kSyncBytes : nullptr, kScratchBytes - kSyncBytes, base);
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
