// C ABI of the multi-head attention forward library (declared in include/mha.h).
//
// Host side only: argument validation (before any launch), workspace carving
// and the three launches of the forward pass, all on the caller's stream.
// Page "Multi-head attention and self-attention", Definition: head i attends
// over (Q W_i^Q, K W_i^K, V W_i^V) and the concatenated heads are multiplied
// by W^O.  Review page "Multi-Head Attention", "The Complete Multi-Head
// Operation": project, attend per head, concatenate, project once more.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <stdint.h>
#include <string.h>

#include "../../include/mha.h"
#include "internal.hpp"

namespace mha {
hipError_t launch_attention_bf16(const AttnParams& p, hipStream_t stream);
hipError_t launch_attention_f16(const AttnParams& p, hipStream_t stream);
hipError_t launch_attention_f32(const AttnParams& p, hipStream_t stream);

hipError_t launch_attention_split_bf16(const AttnParams& p, hipStream_t stream);
hipError_t launch_attention_split_f16(const AttnParams& p, hipStream_t stream);
hipError_t launch_attention_split_f32(const AttnParams& p, hipStream_t stream);
hipError_t launch_split_merge(const AttnParams& p, hipStream_t stream);

hipError_t launch_attention(const AttnParams& p, int elem_dtype, hipStream_t stream) {
  switch (elem_dtype) {
    case kBF16: return launch_attention_bf16(p, stream);
    case kF16: return launch_attention_f16(p, stream);
    case kF32: return launch_attention_f32(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_split(const AttnParams& p, int elem_dtype, hipStream_t stream) {
  hipError_t e;
  switch (elem_dtype) {
    case kBF16: e = launch_attention_split_bf16(p, stream); break;
    case kF16: e = launch_attention_split_f16(p, stream); break;
    case kF32: e = launch_attention_split_f32(p, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_split_merge(p, stream);
}
}  // namespace mha

namespace {

constexpr int64_t kIntMax = 2147483647LL;

size_t esize(int dtype) { return dtype == MHA_F32 ? 4 : 2; }
int vec_elems(int dtype) { return dtype == MHA_F32 ? 4 : 8; }
bool valid_dtype(int dt) { return dt == MHA_F32 || dt == MHA_BF16 || dt == MHA_F16; }
bool valid_work_pair(int in, int work) {
  return (in == MHA_F32 && work == MHA_F32) || (in == MHA_BF16 && work == MHA_F16) ||
         (in == MHA_BF16 && work == MHA_BF16) || (in == MHA_F16 && work == MHA_F16);
}
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Dims used by the attention core: B, h, n_q, n_k, d_h, d_vh, scale, dtypes.
mha_status check_core_dims(const mha_dims* d) {
  if (!d) return MHA_ERR_NULL;
  if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return MHA_ERR_DTYPE;
  if (d->B <= 0 || d->h <= 0 || d->n_q <= 0 || d->n_k <= 0 || d->d_h <= 0 || d->d_vh <= 0)
    return MHA_ERR_DIM;
  if (!isfinite(d->scale)) return MHA_ERR_SCALE;
  // every row index and flattened row count must stay below 2^31
  const int64_t B = d->B, h = d->h;
  if (B * d->n_q > kIntMax || B * d->n_k > kIntMax || B * h * d->n_q > kIntMax ||
      B * h * d->n_k > kIntMax || h * d->d_h > kIntMax || h * d->d_vh > kIntMax)
    return MHA_ERR_DIM;
  if (d->d_h > mha::kMaxHeadDim || d->d_vh > mha::kMaxHeadDim) return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

mha_status check_full_dims(const mha_dims* d) {
  mha_status s = check_core_dims(d);
  if (s != MHA_OK) return s;
  if (!valid_work_pair(d->in_dtype, d->work_dtype)) return MHA_ERR_DTYPE;
  if (d->d_q <= 0 || d->d_k <= 0 || d->d_v <= 0 || d->d_o <= 0) return MHA_ERR_DIM;
  return MHA_OK;
}

mha_status check_mask(const mha_dims* d, const mha_mask* m) {
  if (!m) return MHA_OK;
  const uint32_t known =
      MHA_MASK_CAUSAL | MHA_MASK_KEY_PADDING | MHA_MASK_BOOL | MHA_MASK_ADDITIVE;
  if (m->flags & ~known) return MHA_ERR_MASK;
  if ((m->flags & MHA_MASK_CAUSAL) && d->n_q != d->n_k) return MHA_ERR_MASK;
  if ((m->flags & MHA_MASK_KEY_PADDING) && !m->key_len) return MHA_ERR_MASK;
  if (m->flags & MHA_MASK_BOOL) {
    if (!m->allowed) return MHA_ERR_MASK;
    const int64_t plane = (int64_t)d->n_q * d->n_k;
    if (m->allowed_batch_stride != 0 && m->allowed_batch_stride < plane) return MHA_ERR_MASK;
  }
  if (m->flags & MHA_MASK_ADDITIVE) {
    if (!m->add) return MHA_ERR_MASK;
    const int64_t plane = (int64_t)d->n_q * d->n_k;
    if (m->add_batch_stride != 0 && m->add_batch_stride < plane) return MHA_ERR_MASK;
  }
  if ((m->flags & MHA_MASK_KEY_PADDING) && !aligned(m->key_len, 4)) return MHA_ERR_ALIGN;
  if ((m->flags & MHA_MASK_ADDITIVE) && !aligned(m->add, 4)) return MHA_ERR_ALIGN;
  return MHA_OK;
}

void fill_mask(mha::AttnParams& p, const mha_mask* m) {
  p.causal = 0;
  p.key_len = nullptr;
  p.allowed = nullptr;
  p.allowed_batch_stride = 0;
  p.add = nullptr;
  p.add_batch_stride = 0;
  if (!m) return;
  p.causal = (m->flags & MHA_MASK_CAUSAL) ? 1 : 0;
  if (m->flags & MHA_MASK_KEY_PADDING) p.key_len = m->key_len;
  if (m->flags & MHA_MASK_BOOL) {
    p.allowed = m->allowed;
    p.allowed_batch_stride = m->allowed_batch_stride;
  }
  if (m->flags & MHA_MASK_ADDITIVE) {
    p.add = m->add;
    p.add_batch_stride = m->add_batch_stride;
  }
  p.mask_vec = p.n_k % 4 == 0 && aligned(p.allowed, 4) && p.allowed_batch_stride % 4 == 0 &&
               aligned(p.add, 16) && p.add_batch_stride % 4 == 0;
  p.mask_g16 = p.mask_vec && p.n_k % 16 == 0 && aligned(p.allowed, 16) &&
               p.allowed_batch_stride % 16 == 0 && (int64_t)p.n_q * p.n_k < (int64_t(1) << 31);
}

struct Workspace {
  size_t q, k, v, z, total;
};

// Key partitions of the split form: `requested` > 0 asks for that many
// (fewer if the keys run out: partitions are whole 64-key blocks); 0 lets the
// library choose enough partitions for about 1024 workgroups (four per CU),
// or about 512 for one to four query rows (the decode kernel streams the
// cache: fewer, longer partitions measured 4 % faster at 32768 keys), with
// at least 256 keys each.
struct SplitPlan {
  int splits, split_keys;
  size_t m, l, z, total;   // workspace regions (bytes), 256-byte aligned
};
constexpr int kMaxSplits = 65536;

SplitPlan split_plan(const mha_dims* d, int requested) {
  SplitPlan sp;
  const int64_t n_k = d->n_k;
  int64_t want = requested;
  if (want <= 0) {
    const int64_t base = (int64_t)d->B * d->h * ((d->n_q + 127) / 128);
    const int64_t target = d->n_q <= 4 ? 512 : 1024;
    want = (target + base - 1) / base;
    want = std::min<int64_t>(want, (n_k + 255) / 256);
    if (want < 1) want = 1;
  }
  want = std::min<int64_t>(want, kMaxSplits);
  int64_t keys = (n_k + want - 1) / want;
  keys = (keys + 63) / 64 * 64;
  sp.split_keys = (int)keys;
  sp.splits = (int)((n_k + keys - 1) / keys);
  const size_t rows = (size_t)d->B * d->h * d->n_q;
  sp.m = 0;
  sp.l = round256(sp.splits * rows * 4);
  sp.z = sp.l + round256(sp.splits * rows * 4);
  sp.total = sp.z + round256(sp.splits * rows * (size_t)d->d_vh * 4);
  return sp;
}

// Partition rows (and so workgroups, at most one per partition row) index
// with 32-bit integers.
bool split_plan_fits(const mha_dims* d, const SplitPlan& sp) {
  return (int64_t)sp.splits * d->B * d->h * d->n_q <= kIntMax;
}

Workspace carve(const mha_dims* d) {
  const size_t es = esize(d->work_dtype);
  const size_t B = d->B, h = d->h;
  Workspace w;
  w.q = 0;
  w.k = w.q + round256(B * h * d->n_q * d->d_h * es);
  w.v = w.k + round256(B * h * d->n_k * d->d_h * es);
  w.z = w.v + round256(B * h * d->n_k * d->d_vh * es);
  w.total = w.z + round256(B * d->n_q * h * d->d_vh * es);
  return w;
}

void attn_params(mha::AttnParams& p, const mha_dims* d, int elem_dtype, const void* Qh,
                 const void* Kh, const void* Vh, void* Z, int z_dtype, float* row_m,
                 float* row_l) {
  const int vin = vec_elems(elem_dtype);
  p.Q = Qh;
  p.K = Kh;
  p.V = Vh;
  p.Z = Z;
  p.row_m = row_m;
  p.row_l = row_l;
  p.B = d->B;
  p.h = d->h;
  p.n_q = d->n_q;
  p.n_k = d->n_k;
  p.d_h = d->d_h;
  p.d_vh = d->d_vh;
  p.ldq = d->d_h;
  p.ldk = d->d_h;
  p.ldv = d->d_vh;
  p.ldz = d->h * d->d_vh;
  p.scale_log2 = d->scale * 1.4426950408889634f;
  p.out_dtype = z_dtype;
  p.vec_q = aligned(Qh, 16) && (p.ldq % vin == 0);
  p.vec_k = aligned(Kh, 16) && (p.ldk % vin == 0);
  p.vec_v = aligned(Vh, 16) && (p.ldv % vin == 0);
  p.vec_z = aligned(Z, z_dtype == MHA_F32 ? 16 : 8) && (p.ldz % 4 == 0) && (d->d_vh % 4 == 0);
  p.num_q_tiles = 0;
}

void fill_bwd_mask(mha::AttnBwdParams& p, const mha_mask* m) {
  if (!m) return;
  p.causal = (m->flags & MHA_MASK_CAUSAL) ? 1 : 0;
  if (m->flags & MHA_MASK_KEY_PADDING) p.key_len = m->key_len;
  if (m->flags & MHA_MASK_BOOL) {
    p.allowed = m->allowed;
    p.allowed_batch_stride = m->allowed_batch_stride;
  }
  if (m->flags & MHA_MASK_ADDITIVE) {
    p.add = m->add;
    p.add_batch_stride = m->add_batch_stride;
  }
}

// mha_backward scratch: dZ and the heads' gradients in the concatenated
// layout (work_dtype), the core backward's row terms, column-sum partials.
struct BwdWorkspace {
  size_t dz, dq, dk, dv, lse, dsum, part, splitk, dy, total;
};

BwdWorkspace carve_bwd(const mha_dims* d) {
  const size_t B = d->B, h = d->h, es = esize(d->work_dtype);
  BwdWorkspace w;
  w.dz = 0;
  w.dq = w.dz + round256(B * d->n_q * h * d->d_vh * es);
  w.dk = w.dq + round256(B * d->n_q * h * d->d_h * es);
  w.dv = w.dk + round256(B * d->n_k * h * d->d_h * es);
  w.lse = w.dv + round256(B * d->n_k * h * d->d_vh * es);
  w.dsum = w.lse + round256(B * h * d->n_q * 4);
  w.part = w.dsum + round256(B * h * d->n_q * 4);
  size_t parts = mha::colsum_scratch_floats((int)(B * d->n_q), d->d_o);
  parts = std::max(parts, mha::colsum_scratch_floats((int)(B * d->n_q), (int)(h * d->d_h)));
  parts = std::max(parts, mha::colsum_scratch_floats((int)(B * d->n_k), (int)(h * d->d_h)));
  parts = std::max(parts, mha::colsum_scratch_floats((int)(B * d->n_k), (int)(h * d->d_vh)));
  w.splitk = w.part + round256(parts * 4);
  // split-K partials of the weight gradients (one product at a time)
  const int Mq = (int)(B * d->n_q), Mk = (int)(B * d->n_k);
  const int Nq = (int)(h * d->d_h), Nv = (int)(h * d->d_vh);
  size_t sk = mha::gemm_any_partial_floats(Nv, d->d_o, Mq);
  sk = std::max(sk, mha::gemm_any_partial_floats(d->d_q, Nq, Mq));
  sk = std::max(sk, mha::gemm_any_partial_floats(d->d_k, Nq, Mk));
  sk = std::max(sk, mha::gemm_any_partial_floats(d->d_v, Nv, Mk));
  w.dy = w.splitk + round256(sk * 4);
  // an fp32 dY rounded once to work_dtype for the products that use it (the
  // general product would round it the same way as it stages it)
  const size_t dy_bytes = d->out_dtype == MHA_F32 ? (size_t)Mq * d->d_o * es : 0;
  w.total = w.dy + round256(dy_bytes);
  return w;
}

// Library-owned scratch for attn_core_split_noalloc: the partitions'
// summaries of the key-split form, for callers that cannot allocate.  Every
// GPU the library runs on holds its own copy until the process ends.  In host
// code this name is only a stand-in for the array: the device address comes
// from hipGetSymbolAddress, once per device with that device current, and
// only that address is ever passed to a kernel.
static __device__ __align__(256) char scratch[MHA_STATIC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::atomic<char*> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream), looked up on the first call for that device.
mha_status device_scratch(hipStream_t stream, char** out) {
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return MHA_ERR_LAUNCH;
  dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return MHA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxScratchDevices) return MHA_ERR_LAUNCH;
  char* a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (a == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    a = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (a == nullptr) {
      if (dev != cur && hipSetDevice(dev) != hipSuccess) return MHA_ERR_LAUNCH;
      void* sym = nullptr;
      const hipError_t e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
      if (dev != cur && hipSetDevice(cur) != hipSuccess) return MHA_ERR_LAUNCH;
      if (e != hipSuccess || sym == nullptr) return MHA_ERR_LAUNCH;
      a = static_cast<char*>(sym);
      g_scratch_addr[dev].store(a, std::memory_order_release);
    }
  }
  *out = a;
  return MHA_OK;
}

// Shared body of attn_core_split and attn_core_split_noalloc: checks, then
// the partition and merge launches with the summaries at `ws`.  `ws` is
// NULL for the no-allocation form, which takes the static scratch instead.
mha_status split_forward(const mha_dims* d, const mha_mask* m, const void* Qh, const void* Kh,
                         const void* Vh, void* Z, float* row_m, float* row_l, int32_t splits,
                         void* workspace, size_t workspace_bytes, bool use_scratch,
                         void* stream) {
  mha_status s = check_core_dims(d);
  if (s != MHA_OK) return s;
  if ((s = check_mask(d, m)) != MHA_OK) return s;
  if (splits < 0) return MHA_ERR_DIM;
  if (!Qh || !Kh || !Vh || !Z) return MHA_ERR_NULL;
  const size_t ei = esize(d->in_dtype), eo = esize(d->out_dtype);
  if (!aligned(Qh, ei) || !aligned(Kh, ei) || !aligned(Vh, ei) || !aligned(Z, eo) ||
      !aligned(row_m, 4) || !aligned(row_l, 4))
    return MHA_ERR_ALIGN;
  const SplitPlan sp = split_plan(d, splits);
  if (!split_plan_fits(d, sp)) return MHA_ERR_DIM;
  char* ws = nullptr;
  if (use_scratch) {
    if (sp.total > (size_t)MHA_STATIC_SCRATCH_BYTES) return MHA_ERR_SCRATCH;
    if ((s = device_scratch((hipStream_t)stream, &ws)) != MHA_OK) return s;
  } else {
    if (!workspace || workspace_bytes < sp.total) return MHA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MHA_ERR_ALIGN;
    ws = static_cast<char*>(workspace);
  }
  mha::AttnParams p;
  memset(&p, 0, sizeof(p));
  attn_params(p, d, d->in_dtype, Qh, Kh, Vh, Z, d->out_dtype, row_m, row_l);
  fill_mask(p, m);
  // every (partition, row) summary is written before the merge reads it, so
  // nothing in the scratch needs clearing between calls
  p.splits = sp.splits;
  p.split_keys = sp.split_keys;
  p.part_m = reinterpret_cast<float*>(ws + sp.m);
  p.part_l = reinterpret_cast<float*>(ws + sp.l);
  p.part_z = reinterpret_cast<float*>(ws + sp.z);
  if (mha::launch_attention_split(p, d->in_dtype, (hipStream_t)stream) != hipSuccess)
    return MHA_ERR_LAUNCH;
  return MHA_OK;
}

}  // namespace

extern "C" {

size_t mha_workspace_bytes(const mha_dims* d) {
  if (check_full_dims(d) != MHA_OK) return 0;
  return carve(d).total;
}

int32_t mha_max_head_dim(void) { return mha::kMaxHeadDim; }

const char* mha_status_string(int s) {
  switch (s) {
    case MHA_OK: return "MHA_OK";
    case MHA_ERR_NULL: return "MHA_ERR_NULL: a required pointer is NULL";
    case MHA_ERR_DIM: return "MHA_ERR_DIM: a dimension is not positive or is too large";
    case MHA_ERR_DTYPE: return "MHA_ERR_DTYPE: unknown element type";
    case MHA_ERR_MASK: return "MHA_ERR_MASK: invalid mask descriptor";
    case MHA_ERR_ALIGN: return "MHA_ERR_ALIGN: a pointer is misaligned for its element type";
    case MHA_ERR_WORKSPACE: return "MHA_ERR_WORKSPACE: workspace missing or too small";
    case MHA_ERR_UNSUPPORTED: return "MHA_ERR_UNSUPPORTED: head width above the instantiated maximum";
    case MHA_ERR_LAUNCH: return "MHA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    case MHA_ERR_SCALE: return "MHA_ERR_SCALE: the score scale is not finite";
    case MHA_ERR_SCRATCH:
      return "MHA_ERR_SCRATCH: the partitions' summaries need more than the library's static "
             "scratch (MHA_STATIC_SCRATCH_BYTES); use fewer splits or attn_core_split";
    default: return "unknown mha_status";
  }
}

mha_status attn_core(const mha_dims* d, const mha_mask* m, const void* Qh, const void* Kh,
                     const void* Vh, void* Z, float* row_m, float* row_l, void* stream) {
  mha_status s = check_core_dims(d);
  if (s != MHA_OK) return s;
  if ((s = check_mask(d, m)) != MHA_OK) return s;
  if (!Qh || !Kh || !Vh || !Z) return MHA_ERR_NULL;
  const size_t ei = esize(d->in_dtype), eo = esize(d->out_dtype);
  if (!aligned(Qh, ei) || !aligned(Kh, ei) || !aligned(Vh, ei) || !aligned(Z, eo) ||
      !aligned(row_m, 4) || !aligned(row_l, 4))
    return MHA_ERR_ALIGN;
  mha::AttnParams p;
  memset(&p, 0, sizeof(p));
  attn_params(p, d, d->in_dtype, Qh, Kh, Vh, Z, d->out_dtype, row_m, row_l);
  fill_mask(p, m);
  if (mha::launch_attention(p, d->in_dtype, (hipStream_t)stream) != hipSuccess)
    return MHA_ERR_LAUNCH;
  return MHA_OK;
}

size_t attn_split_workspace_bytes(const mha_dims* d, int32_t splits) {
  if (check_core_dims(d) != MHA_OK || splits < 0) return 0;
  const SplitPlan sp = split_plan(d, splits);
  if (!split_plan_fits(d, sp)) return 0;
  return sp.total;
}

mha_status attn_core_split(const mha_dims* d, const mha_mask* m, const void* Qh, const void* Kh,
                           const void* Vh, void* Z, float* row_m, float* row_l, int32_t splits,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return split_forward(d, m, Qh, Kh, Vh, Z, row_m, row_l, splits, workspace, workspace_bytes,
                       false, stream);
}

mha_status attn_core_split_noalloc(const mha_dims* d, const mha_mask* m, const void* Qh,
                                   const void* Kh, const void* Vh, void* Z, float* row_m,
                                   float* row_l, int32_t splits, void* stream) {
  return split_forward(d, m, Qh, Kh, Vh, Z, row_m, row_l, splits, nullptr, 0, true, stream);
}

size_t attn_backward_workspace_bytes(const mha_dims* d) {
  if (check_core_dims(d) != MHA_OK) return 0;
  return 2 * round256((size_t)d->B * d->h * d->n_q * 4);
}

// Checks shared by attn_core_backward and attn_bias_backward, and the
// kernels' parameters (dQ, dK, dV left NULL).
mha_status core_backward_params(const mha_dims* d, const mha_mask* m, const void* Qh,
                                const void* Kh, const void* Vh, const void* Z, const void* dZ,
                                const float* row_m, const float* row_l, void* workspace,
                                size_t workspace_bytes, mha::AttnBwdParams& p) {
  mha_status s = check_core_dims(d);
  if (s != MHA_OK) return s;
  if ((s = check_mask(d, m)) != MHA_OK) return s;
  if (!Qh || !Kh || !Vh || !Z || !dZ || !row_m || !row_l) return MHA_ERR_NULL;
  const size_t ei = esize(d->in_dtype), eo = esize(d->out_dtype);
  if (!aligned(Qh, ei) || !aligned(Kh, ei) || !aligned(Vh, ei) || !aligned(Z, eo) ||
      !aligned(dZ, eo) || !aligned(row_m, 4) || !aligned(row_l, 4))
    return MHA_ERR_ALIGN;
  const size_t rows = (size_t)d->B * d->h * d->n_q;
  if (!workspace || workspace_bytes < attn_backward_workspace_bytes(d)) return MHA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MHA_ERR_ALIGN;
  memset(&p, 0, sizeof(p));
  p.Q = Qh;
  p.K = Kh;
  p.V = Vh;
  p.Z = Z;
  p.dZ = dZ;
  p.row_m = row_m;
  p.row_l = row_l;
  p.lse2 = static_cast<float*>(workspace);
  p.dsum = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256(rows * 4));
  p.B = d->B;
  p.h = d->h;
  p.n_q = d->n_q;
  p.n_k = d->n_k;
  p.d_h = d->d_h;
  p.d_vh = d->d_vh;
  p.ldz = d->h * d->d_vh;
  p.scale = d->scale;
  p.scale_log2 = d->scale * 1.4426950408889634f;
  p.elem_dtype = d->in_dtype;
  p.z_dtype = d->out_dtype;
  p.g_dtype = d->out_dtype;
  fill_bwd_mask(p, m);
  const int vin = vec_elems(d->in_dtype), vz = vec_elems(d->out_dtype);
  p.vec_q = aligned(Qh, 16) && d->d_h % vin == 0;
  p.vec_k = aligned(Kh, 16) && d->d_h % vin == 0;
  p.vec_v = aligned(Vh, 16) && d->d_vh % vin == 0;
  p.vec_z = aligned(dZ, 16) && aligned(Z, 16) && d->d_vh % vz == 0;
  return MHA_OK;
}

mha_status attn_core_backward(const mha_dims* d, const mha_mask* m, const void* Qh,
                              const void* Kh, const void* Vh, const void* Z, const void* dZ,
                              const float* row_m, const float* row_l, void* dQh, void* dKh,
                              void* dVh, void* workspace, size_t workspace_bytes, void* stream) {
  mha::AttnBwdParams p;
  mha_status s = core_backward_params(d, m, Qh, Kh, Vh, Z, dZ, row_m, row_l, workspace,
                                      workspace_bytes, p);
  if (s != MHA_OK) return s;
  if (!dQh || !dKh || !dVh) return MHA_ERR_NULL;
  const size_t eo = esize(d->out_dtype);
  if (!aligned(dQh, eo) || !aligned(dKh, eo) || !aligned(dVh, eo)) return MHA_ERR_ALIGN;
  p.dQ = dQh;
  p.dK = dKh;
  p.dV = dVh;
  const size_t a4 = 4 * eo;   // four-element stores
  p.vec_dq = aligned(dQh, a4) && d->d_h % 4 == 0;
  p.vec_dk = aligned(dKh, a4) && d->d_h % 4 == 0;
  p.vec_dv = aligned(dVh, a4) && d->d_vh % 4 == 0;
  if (mha::launch_attention_backward(p, d->in_dtype, (hipStream_t)stream) != hipSuccess)
    return MHA_ERR_LAUNCH;
  return MHA_OK;
}

mha_status attn_bias_backward(const mha_dims* d, const mha_mask* m, const void* Qh,
                              const void* Kh, const void* Vh, const void* Z, const void* dZ,
                              const float* row_m, const float* row_l, float* dM,
                              void* workspace, size_t workspace_bytes, void* stream) {
  mha::AttnBwdParams p;
  mha_status s = core_backward_params(d, m, Qh, Kh, Vh, Z, dZ, row_m, row_l, workspace,
                                      workspace_bytes, p);
  if (s != MHA_OK) return s;
  if (!m || !(m->flags & MHA_MASK_ADDITIVE)) return MHA_ERR_MASK;
  if (!dM) return MHA_ERR_NULL;
  if (!aligned(dM, 4)) return MHA_ERR_ALIGN;
  const int shared = (m->add_batch_stride == 0) ? 1 : 0;
  hipStream_t st = (hipStream_t)stream;
  if (mha::launch_bwd_row_terms(p, st) != hipSuccess) return MHA_ERR_LAUNCH;
  if (mha::launch_bias_backward(p, dM, shared, st) != hipSuccess) return MHA_ERR_LAUNCH;
  return MHA_OK;
}

size_t mha_backward_workspace_bytes(const mha_dims* d) {
  if (check_full_dims(d) != MHA_OK) return 0;
  return carve_bwd(d).total;
}

mha_status mha_backward(const mha_dims* d, const mha_mask* m, const void* Q, const void* K,
                        const void* V, const void* W_Q, const void* W_K, const void* W_V,
                        const void* W_O, const void* dY, const float* row_m, const float* row_l,
                        const void* fwd_workspace, size_t fwd_workspace_bytes, void* dQ,
                        void* dK, void* dV, void* dW_Q, void* dW_K, void* dW_V, void* dW_O,
                        const mha_bias_grad* dbias, void* workspace, size_t workspace_bytes,
                        void* stream) {
  mha_status s = check_full_dims(d);
  if (s != MHA_OK) return s;
  if ((s = check_mask(d, m)) != MHA_OK) return s;
  if (!Q || !K || !V || !W_Q || !W_K || !W_V || !W_O || !dY || !row_m || !row_l ||
      !fwd_workspace)
    return MHA_ERR_NULL;
  const size_t ei = esize(d->in_dtype), eo = esize(d->out_dtype);
  const mha_bias_grad nb = {nullptr, nullptr, nullptr, nullptr};
  const mha_bias_grad& db = dbias ? *dbias : nb;
  if (!aligned(Q, ei) || !aligned(K, ei) || !aligned(V, ei) || !aligned(W_Q, ei) ||
      !aligned(W_K, ei) || !aligned(W_V, ei) || !aligned(W_O, ei) || !aligned(dY, eo) ||
      !aligned(row_m, 4) || !aligned(row_l, 4) || !aligned(dQ, eo) || !aligned(dK, eo) ||
      !aligned(dV, eo) || !aligned(dW_Q, eo) || !aligned(dW_K, eo) || !aligned(dW_V, eo) ||
      !aligned(dW_O, eo) || !aligned(db.db_Q, eo) || !aligned(db.db_K, eo) ||
      !aligned(db.db_V, eo) || !aligned(db.db_O, eo))
    return MHA_ERR_ALIGN;
  const Workspace fw = carve(d);
  if (fwd_workspace_bytes < fw.total) return MHA_ERR_WORKSPACE;
  if (!aligned(fwd_workspace, 256)) return MHA_ERR_ALIGN;
  const BwdWorkspace bw = carve_bwd(d);
  if (!workspace || workspace_bytes < bw.total) return MHA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MHA_ERR_ALIGN;

  const char* fws = static_cast<const char*>(fwd_workspace);
  char* ws = static_cast<char*>(workspace);
  const int wd = d->work_dtype, od = d->out_dtype, id = d->in_dtype;
  const int Mq = d->B * d->n_q, Mk = d->B * d->n_k;
  const int Nq = d->h * d->d_h, Nv = d->h * d->d_vh;
  float* part = reinterpret_cast<float*>(ws + bw.part);
  hipStream_t st = (hipStream_t)stream;
  auto gemm = [&](const void* A, int adt, long long lda, int at, const void* W, int wdt,
                  long long ldw, int wt, void* C, int M, int N, int Kd) {
    mha::GemmAny g;
    memset(&g, 0, sizeof(g));
    g.A = A;
    g.W = W;
    g.C = C;
    g.M = M;
    g.N = N;
    g.K = Kd;
    g.lda = lda;
    g.ldw = ldw;
    g.ldc = N;
    g.a_trans = at;
    g.w_trans = wt;
    g.a_dtype = adt;
    g.w_dtype = wdt;
    g.c_dtype = C == ws + bw.dz ? wd : od;
    return mha::launch_gemm_any(g, wd, reinterpret_cast<float*>(ws + bw.splitk), st) ==
           hipSuccess;
  };

  // output projection: dZ = dY W_O^T (W_O [Nv, d_o] is W_O^T stored k-contiguous),
  // dW_O = Z^T dY, db_O = column sums of dY (of dY as given)
  void* dZ = ws + bw.dz;
  const void* dYp = dY;
  int dydt = od;
  if (od == MHA_F32 && wd != MHA_F32) {
    if (mha::launch_round_f32(static_cast<const float*>(dY), ws + bw.dy, (size_t)Mq * d->d_o, wd,
                              st) != hipSuccess)
      return MHA_ERR_LAUNCH;
    dYp = ws + bw.dy;
    dydt = wd;
  }
  if (!gemm(dYp, dydt, d->d_o, 0, W_O, id, d->d_o, 1, dZ, Mq, Nv, d->d_o)) return MHA_ERR_LAUNCH;
  if (dW_O && !gemm(fws + fw.z, wd, Nv, 1, dYp, dydt, d->d_o, 0, dW_O, Nv, d->d_o, Mq))
    return MHA_ERR_LAUNCH;
  if (db.db_O && mha::launch_colsum(dY, od, d->d_o, Mq, d->d_o, db.db_O, od, part, st) != hipSuccess)
    return MHA_ERR_LAUNCH;

  // the core backward, gradients in the concatenated layout
  mha::AttnBwdParams p;
  memset(&p, 0, sizeof(p));
  p.Q = fws + fw.q;
  p.K = fws + fw.k;
  p.V = fws + fw.v;
  p.Z = fws + fw.z;
  p.dZ = dZ;
  p.row_m = row_m;
  p.row_l = row_l;
  p.dQ = ws + bw.dq;
  p.dK = ws + bw.dk;
  p.dV = ws + bw.dv;
  p.lse2 = reinterpret_cast<float*>(ws + bw.lse);
  p.dsum = reinterpret_cast<float*>(ws + bw.dsum);
  p.B = d->B;
  p.h = d->h;
  p.n_q = d->n_q;
  p.n_k = d->n_k;
  p.d_h = d->d_h;
  p.d_vh = d->d_vh;
  p.ldz = Nv;
  p.scale = d->scale;
  p.scale_log2 = d->scale * 1.4426950408889634f;
  p.grad_concat = 1;
  p.elem_dtype = wd;
  p.z_dtype = wd;
  p.g_dtype = wd;
  fill_bwd_mask(p, m);
  p.vec_q = p.vec_k = (d->d_h % 8 == 0);      // workspace regions are 256-byte aligned
  p.vec_v = (d->d_vh % 8 == 0);
  p.vec_z = (d->d_vh % 8 == 0);
  p.vec_dq = p.vec_dk = (d->d_h % 4 == 0);
  p.vec_dv = (d->d_vh % 4 == 0);
  if (mha::launch_attention_backward(p, wd, st) != hipSuccess) return MHA_ERR_LAUNCH;

  // projections: dW = X^T dX_cat, db = column sums of dX_cat, dX = dX_cat W^T
  struct Proj {
    const void* X; int M, d_in; const void* W; int N; const char* cat;
    void* dX; void* dW; void* db;
  };
  const Proj proj[3] = {
      {Q, Mq, d->d_q, W_Q, Nq, ws + bw.dq, dQ, dW_Q, db.db_Q},
      {K, Mk, d->d_k, W_K, Nq, ws + bw.dk, dK, dW_K, db.db_K},
      {V, Mk, d->d_v, W_V, Nv, ws + bw.dv, dV, dW_V, db.db_V},
  };
  for (const Proj& r : proj) {
    if (r.dW && !gemm(r.X, id, r.d_in, 1, r.cat, wd, r.N, 0, r.dW, r.d_in, r.N, r.M))
      return MHA_ERR_LAUNCH;
    if (r.db && mha::launch_colsum(r.cat, wd, r.N, r.M, r.N, r.db, od, part, st) != hipSuccess)
      return MHA_ERR_LAUNCH;
    if (r.dX && !gemm(r.cat, wd, r.N, 0, r.W, id, r.N, 1, r.dX, r.M, r.d_in, r.N))
      return MHA_ERR_LAUNCH;
  }
  return MHA_OK;
}

mha_status mha_forward(const mha_dims* d, const mha_mask* m, const void* Q, const void* K,
                       const void* V, const void* W_Q, const void* W_K, const void* W_V,
                       const void* W_O, const mha_bias* bias, void* Y, float* row_m,
                       float* row_l, void* workspace, size_t workspace_bytes, void* stream) {
  mha_status s = check_full_dims(d);
  if (s != MHA_OK) return s;
  if ((s = check_mask(d, m)) != MHA_OK) return s;
  if (!Q || !K || !V || !W_Q || !W_K || !W_V || !W_O || !Y) return MHA_ERR_NULL;
  const size_t ei = esize(d->in_dtype), eo = esize(d->out_dtype);
  if (!aligned(Q, ei) || !aligned(K, ei) || !aligned(V, ei) || !aligned(W_Q, ei) ||
      !aligned(W_K, ei) || !aligned(W_V, ei) || !aligned(W_O, ei) || !aligned(Y, eo) ||
      !aligned(row_m, 4) || !aligned(row_l, 4))
    return MHA_ERR_ALIGN;
  const mha_bias nb = {nullptr, nullptr, nullptr, nullptr};
  const mha_bias& bs = bias ? *bias : nb;
  if (!aligned(bs.b_Q, ei) || !aligned(bs.b_K, ei) || !aligned(bs.b_V, ei) ||
      !aligned(bs.b_O, ei))
    return MHA_ERR_ALIGN;
  const Workspace w = carve(d);
  if (!workspace || workspace_bytes < w.total) return MHA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MHA_ERR_ALIGN;

  char* ws = static_cast<char*>(workspace);
  void* Qh = ws + w.q;
  void* Kh = ws + w.k;
  void* Vh = ws + w.v;
  void* Z = ws + w.z;
  const int vin = vec_elems(d->in_dtype);
  const int vwork = vec_elems(d->work_dtype);
  hipStream_t st = (hipStream_t)stream;

  // K1: the three head projections in one launch, stored head-major.
  mha::GemmBatch gb;
  memset(&gb, 0, sizeof(gb));
  gb.count = 3;
  const void* srcs[3] = {Q, K, V};
  const void* ws3[3] = {W_Q, W_K, W_V};
  const void* b3[3] = {bs.b_Q, bs.b_K, bs.b_V};
  void* dst[3] = {Qh, Kh, Vh};
  const int Ms[3] = {d->B * d->n_q, d->B * d->n_k, d->B * d->n_k};
  const int Ks[3] = {d->d_q, d->d_k, d->d_v};
  const int dhs[3] = {d->d_h, d->d_h, d->d_vh};
  const int ntoks[3] = {d->n_q, d->n_k, d->n_k};
  for (int i = 0; i < 3; ++i) {
    mha::GemmProblem& p = gb.p[i];
    p.A = srcs[i];
    p.W = ws3[i];
    p.C = dst[i];
    p.M = Ms[i];
    p.N = d->h * dhs[i];
    p.K = Ks[i];
    p.epilogue = mha::kHeads;
    p.out_dtype = d->work_dtype;
    p.heads = d->h;
    p.dh = dhs[i];
    p.ntok = ntoks[i];
    p.vec_a = aligned(p.A, 16) && (p.K % vin == 0);
    p.vec_w = aligned(p.W, 16) && (p.N % vin == 0);
    p.vec_c = 1;
    p.bias = b3[i];
  }
  if (mha::launch_gemm(gb, d->in_dtype, d->in_dtype, st) != hipSuccess) return MHA_ERR_LAUNCH;

  // K2: fused attention, written into the concatenation Z (work_dtype).
  mha::AttnParams ap;
  memset(&ap, 0, sizeof(ap));
  attn_params(ap, d, d->work_dtype, Qh, Kh, Vh, Z, d->work_dtype, row_m, row_l);
  fill_mask(ap, m);
  if (mha::launch_attention(ap, d->work_dtype, st) != hipSuccess) return MHA_ERR_LAUNCH;

  // K3: Y = Z W^O, row-major.
  mha::GemmBatch ob;
  memset(&ob, 0, sizeof(ob));
  ob.count = 1;
  mha::GemmProblem& o = ob.p[0];
  o.A = Z;
  o.W = W_O;
  o.C = Y;
  o.M = d->B * d->n_q;
  o.N = d->d_o;
  o.K = d->h * d->d_vh;
  o.epilogue = mha::kRowMajor;
  o.out_dtype = d->out_dtype;
  o.bias = bs.b_O;
  o.vec_a = (o.K % vwork == 0);
  o.vec_w = aligned(W_O, 16) && (o.N % vin == 0);
  o.vec_c = aligned(Y, 16);
  if (mha::launch_gemm(ob, d->work_dtype, d->in_dtype, st) != hipSuccess) return MHA_ERR_LAUNCH;
  return MHA_OK;
}

}  // extern "C"
